// Decode attention: sequences with exactly one new token read all of their
// cached K/V through the block table; HBM-bound ("Inside vLLM", section
// "Scheduler": decode steps are memory-bandwidth-bound; ngrok "Serving models
// at scale with vLLM", section "Speculative decoding": a decode pass is
// limited by moving data, not by math).
//
// Design for gfx950 (the pages give no kernel design):
//  - A workgroup owns (sequence s, KV head g, partition p), the keys
//    [p * PT, min((p + 1) * PT, L)). Its 4 waves take the partition's 16-token
//    blocks round-robin, so neighbouring waves stream neighbouring blocks,
//    and merge their partial softmax states through LDS at the end. All
//    G = Hq / Hkv query heads of the group share each K/V read.
//  - Scores use MFMA with the key rows as the A operand: S^T = K . Q^T. Each
//    lane loads the 16-byte K chunk it feeds the matrix core straight from
//    HBM. Query heads fill the 16 columns (G <= 16; unused columns are zero
//    and cost nothing in an HBM-bound kernel).
//  - In the score layout a lane holds one head column and 4 consecutive key
//    rows, which is already the P^T operand of the 16x16x16 bf16 MFMA. V needs
//    keys contiguous per lane instead of d, so each wave transposes its block
//    of V through a private LDS tile (8-byte writes and reads, no barrier),
//    and O^T = V^T . P^T runs in bf16 with fp32 accumulation. Each lane then
//    owns one head column of O^T, so rescaling needs no lane exchange.
//    fp32 inputs keep an exact path: V widened, P.V on the fp32 16x16x4 MFMA.
//  - Online softmax in log2 units with a lazy rescale: the running maximum is
//    only raised (and the accumulators rescaled) when a block's maximum beats
//    it by more than 2^8, so weights stay <= 256 and rescales are rare.
//  - Each wave can keep NPF blocks of K and V in flight in registers (a ring
//    of static slots). One slot measures best: the occupancy it leaves hides
//    HBM latency better than deeper rings.
//  - Sequences longer than one partition write (unnormalised output, max,
//    weight sum) per partition; a second kernel combines partitions in a fixed
//    order (deterministic). Single-partition sequences write the output
//    directly.
#include <cstdlib>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr int kVtRow = 20;                 // bf16 elements per row of a wave's V^T tile (16 keys + pad)

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
  static constexpr int KC = D * ES / 64;           // 16-byte K chunks per lane per block
  static constexpr int VE = D / 16;                // V elements per lane per row
  static constexpr int VW = VE * ES / 4;           // 32-bit words per lane per V row
  static constexpr int NACC = BF16 ? D / 16 : VE;  // 16x16 accumulator tiles
  static constexpr int VT_BYTES = BF16 ? D * kVtRow * 2 : 0;  // per-wave V^T tile
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

// Consume one block: scores, online softmax, P.V. `blk` is the block's index
// within the sequence; rows at or past `end` are masked. Lane (kg, n) holds
// K row n and V rows 4kg..4kg+3 (elements VE*n..VE*n+VE-1) of the block.
// Accumulators: bf16 path O^T[d = 16t + 4kg + r][head n] in o[t][r];
// fp32 path O[head 4kg + r][d = VE*n + e] in o[e][r].
template <bool BF16, int D>
__device__ inline void attend_block(BlockRegs<BF16, D>& cur, const uint4 (&qv)[DecodeShape<BF16, D>::KC],
                                    f32x4 (&o)[DecodeShape<BF16, D>::NACC], float& m_run, float& l_run,
                                    uint16_t* vt, int blk, int end, int kg, int n, float qk_scale) {
  using Sh = DecodeShape<BF16, D>;
  constexpr int KC = Sh::KC, VE = Sh::VE, VW = Sh::VW;
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
  const int tok0 = blk * kBlockTokens + 4 * kg;
#pragma unroll
  for (int r = 0; r < 4; ++r) sc[r] = (tok0 + r < end) ? acc[r] * qk_scale : -INFINITY;
  float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  if (__any(mloc > m_run + kRescaleThreshold)) {
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = fast_exp2(m_run - m_new);
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
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pr[r] = fast_exp2(sc[r] - m_run);
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
    // V^T tile: vt[d][key], keys 4kg..4kg+3 of column d in one 8-byte word.
#pragma unroll
    for (int w = 0; w < VW; ++w) {
      const uint32_t v0 = cur.v[0][w], v1 = cur.v[1][w], v2 = cur.v[2][w], v3 = cur.v[3][w];
      const int d = VE * n + 2 * w;
      *reinterpret_cast<uint2*>(vt + d * kVtRow + 4 * kg) =
          make_uint2((v0 & 0xffffu) | (v1 << 16), (v2 & 0xffffu) | (v3 << 16));
      *reinterpret_cast<uint2*>(vt + (d + 1) * kVtRow + 4 * kg) =
          make_uint2((v0 >> 16) | (v1 & 0xffff0000u), (v2 >> 16) | (v3 & 0xffff0000u));
    }
    __builtin_amdgcn_wave_barrier();
    const i16x4 pb = __builtin_bit_cast(i16x4, make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])));
#pragma unroll
    for (int t = 0; t < Sh::NACC; ++t) {
      const i16x4 va =
          __builtin_bit_cast(i16x4, *reinterpret_cast<const uint2*>(vt + (16 * t + n) * kVtRow + 4 * kg));
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

// Grid: x = sequence * Hkv + KV head, y = partition. Dynamic LDS: per-wave V^T
// tiles during the sweep, then each wave's (max, sum, output) for the merge.
template <bool BF16, int D, int NPF>
__global__ __launch_bounds__(kThreads) void decode_kernel(AttnArgs a) {
  using Sh = DecodeShape<BF16, D>;
  constexpr int ES = Sh::ES, KC = Sh::KC, VE = Sh::VE;
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // K row (token) for the A operand; head column of scores
  const int kg = lane >> 4;  // lane group: token rows 4kg..4kg+3 of scores
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t Hkv = static_cast<uint32_t>(a.Hkv);
  const uint32_t s = blockIdx.x / Hkv, g = blockIdx.x - s * Hkv;
  const int p = blockIdx.y;
  const int q0 = a.qsl[s], q1 = a.qsl[s + 1];
  if (q1 - q0 != 1 || q0 < 0 || q0 >= a.T) return;  // decode sequences only (whole workgroup)
  const int PT = static_cast<int>(a.part_tokens);
  const int L = static_cast<int>(min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens));
  const int start = p * PT;
  if (start >= L) return;  // whole workgroup
  const int end = min(start + PT, L);
  const int nparts = (L + PT - 1) / PT;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  const float qk_scale = a.scale * kLog2e;
  const int b0 = start / kBlockTokens;
  const int nblk = (end - start + kBlockTokens - 1) / kBlockTokens;
  const int nbw = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;  // blocks b0 + wave + 4i

  // Q^T as the B operand: lane (kg, n) holds head n, the same d positions its
  // K chunks cover. Columns n >= G are zero.
  uint4 qv[KC];
  {
    const char* qrow = a.q + int64_t(q0) * a.q_st + int64_t(g * G + n) * a.q_sh + 16 * kg;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qv[c] = n < G ? *reinterpret_cast<const uint4*>(qrow + 64 * c) : make_uint4(0, 0, 0, 0);
  }

  const int32_t* bt = a.block_tables + int64_t(s) * a.bt_row;
  const char* kbase = a.kc + int64_t(g) * a.kc_sh + n * a.kc_sr + 16 * kg;
  const char* vbase = a.vc + int64_t(g) * a.vc_sh + (4 * kg) * a.vc_sr + VE * ES * n;
  const uint32_t NB = static_cast<uint32_t>(min(a.NB, int64_t(0x7fffffff)));
  auto load = [&](BlockRegs<BF16, D>& r, int i) {
    const uint32_t id = static_cast<uint32_t>(bt[b0 + wave + kWaves * i]);
    const int64_t pid = id < NB ? int64_t(id) : 0;
    load_block<BF16, D>(r, kbase + pid * a.kc_sb, vbase + pid * a.vc_sb, a.vc_sr);
  };
  uint16_t* vt = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(smem) + wave * Sh::VT_BYTES);

  f32x4 o[Sh::NACC];
#pragma unroll
  for (int t = 0; t < Sh::NACC; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  BlockRegs<BF16, D> ring[NPF];
#pragma unroll
  for (int j = 0; j < NPF; ++j)
    if (j < nbw) load(ring[j], j);
  for (int i = 0; i < nbw; i += NPF) {
#pragma unroll
    for (int j = 0; j < NPF; ++j) {
      const int ib = i + j;
      if (ib < nbw) {
        attend_block<BF16, D>(ring[j], qv, o, m_run, l_run, vt, b0 + wave + kWaves * ib, end, kg, n, qk_scale);
        if (ib + NPF < nbw) load(ring[j], ib + NPF);
      }
    }
  }

  // merge the 4 waves: LDS layout [wave][m: 16][l: 16][o: G * D]
  __syncthreads();  // V^T tiles are no longer in use
  const int wstride = 32 + G * D;
  float* ws = smem + wave * wstride;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (kg == 0) {
    ws[n] = m_run;
    ws[16 + n] = l_tot;
  }
  if constexpr (BF16) {
    if (n < G) {
#pragma unroll
      for (int t = 0; t < Sh::NACC; ++t)
        *reinterpret_cast<float4*>(ws + 32 + n * D + 16 * t + 4 * kg) =
            make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * kg + r;
      if (h < G) {
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(ws + 32 + h * D + VE * n + e) =
              make_float4(o[e][r], o[e + 1][r], o[e + 2][r], o[e + 3][r]);
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += kThreads) {
    const int h = idx / (D / 4), d = 4 * (idx - h * (D / 4));
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, smem[w * wstride + h]);
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* wsw = smem + w * wstride;
      const float sw = fast_exp2(wsw[h] - m);  // 0 for a wave that saw no block
      lsum += sw * wsw[16 + h];
      const float4 x = *reinterpret_cast<const float4*>(wsw + 32 + h * D + d);
      acc.x += sw * x.x;
      acc.y += sw * x.y;
      acc.z += sw * x.z;
      acc.w += sw * x.w;
    }
    const int64_t hq = int64_t(g) * G + h;
    if (nparts == 1) {
      const float inv = 1.f / lsum;
      char* dst = a.out + int64_t(q0) * a.out_st + hq * a.out_sh + d * ES;
      if constexpr (BF16) {
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      }
    } else {
      const int64_t slot = (int64_t(s) * a.Hq + hq) * a.max_parts + p;
      *reinterpret_cast<float4*>(a.ws_o + slot * D + d) = acc;
      if (d == 0) a.ws_ml[slot] = make_float2(m, lsum);
    }
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
  const int64_t s = item / a.Hq, hq = item - s * a.Hq;
  if (s >= a.S) return;
  const int q0 = a.qsl[s], q1 = a.qsl[s + 1];
  if (q1 - q0 != 1 || q0 < 0 || q0 >= a.T) return;
  const int64_t L = min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens);
  const int nparts = static_cast<int>((L + a.part_tokens - 1) / a.part_tokens);
  if (nparts <= 1) return;
  const float2* ml = a.ws_ml + (s * a.Hq + hq) * a.max_parts;
  const float* po = a.ws_o + (s * a.Hq + hq) * a.max_parts * D + DPL * lane;
  float m = -INFINITY;
  for (int p = lane; p < nparts; p += 64) m = fmaxf(m, ml[p].x);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float acc[DPL] = {};
  float lsum = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    float w = 0.f;
    if (p0 + lane < nparts) {
      const float2 v = ml[p0 + lane];
      w = fast_exp2(v.x - m);
      lsum += w * v.y;
    }
    const int cnt = min(64, nparts - p0);
    for (int j = 0; j < cnt; ++j) {
      const float wj = __shfl(w, j);
      const float* x = po + int64_t(p0 + j) * D;
      if constexpr (DPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(x);
        acc[0] += wj * v.x;
        acc[1] += wj * v.y;
      } else {
        acc[0] += wj * x[0];
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
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

template <bool BF16, int D, int NPF>
hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
  using Sh = DecodeShape<BF16, D>;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  const size_t merge = sizeof(float) * kWaves * (32 + G * D);
  const size_t tiles = size_t(kWaves) * Sh::VT_BYTES;
  const size_t lds = merge > tiles ? merge : tiles;
  const dim3 grid(static_cast<unsigned>(a.S * a.Hkv), static_cast<unsigned>(a.max_parts));
  {
    ProfileScope ps(kDecode, stream);
    hipLaunchKernelGGL((decode_kernel<BF16, D, NPF>), grid, dim3(kThreads), lds, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const int64_t rblocks = (a.S * a.Hq + kWaves - 1) / kWaves;
  {
    ProfileScope ps(kReduce, stream);
    hipLaunchKernelGGL((reduce_kernel<BF16, D>), dim3(static_cast<unsigned>(rblocks)), dim3(kThreads), 0, stream,
                       a);
  }
  return hipGetLastError();
}

int prefetch_depth() {
  static const int forced = [] {
    const char* e = std::getenv("PA_DECODE_PREFETCH");
    return e ? std::atoi(e) : 0;
  }();
  return (forced >= 1 && forced <= 3) ? forced : 1;
}

template <bool BF16, int D>
hipError_t launch_depth(const AttnArgs& a, hipStream_t stream) {
  switch (prefetch_depth()) {
    case 2: return launch_typed<BF16, D, 2>(a, stream);
    case 3: return launch_typed<BF16, D, 3>(a, stream);
    default: return launch_typed<BF16, D, 1>(a, stream);
  }
}

}  // namespace

hipError_t launch_decode(const AttnArgs& a, hipStream_t stream) {
  const bool bf16 = a.elem == Elem::BF16;
  if (a.D == 64) return bf16 ? launch_depth<true, 64>(a, stream) : launch_depth<false, 64>(a, stream);
  return bf16 ? launch_depth<true, 128>(a, stream) : launch_depth<false, 128>(a, stream);
}

}  // namespace pa
