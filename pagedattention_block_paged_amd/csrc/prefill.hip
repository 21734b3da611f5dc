// Chunked-prefill attention: sequences with more than one new token. Query i
// of a chunk that follows C cached tokens sits at position C + i and sees keys
// 0 .. C + i: the whole cached context plus the chunk's own earlier tokens
// (ngrok "Serving models at scale with vLLM", section "Chunked prefill": a
// later chunk reads the earlier chunks' K/V from the cache, and a token
// depends only on the tokens before it). A dense contraction, compute-bound
// ("Inside vLLM", section "Scheduler": prefill is usually compute-bound).
//
// Design for gfx950 (the pages give no kernel design):
//  - A plan kernel lists the q-tiles of every prefill sequence (exclusive
//    prefix sum of tiles per sequence), so the host never reads lengths.
//  - A workgroup of 4 waves owns one (q-tile, KV head, group of HW query
//    heads); wave w takes query head hw = w % HW and 32 tokens of sub-tile
//    w / HW. The 4 waves share K/V tiles of 64 keys staged in LDS: K row-major,
//    V transposed ([d][key]) while staging, so both matrix-core operands are
//    read with plain vector LDS reads.
//  - S^T = K . Q^T with 32x32 MFMA (bf16: 32x32x16). With keys as rows, each
//    lane owns one query token: the row max needs one cross-lane exchange, the
//    rescale of the output accumulators needs none, and the scores are already
//    laid out as the B operand of O^T = V^T . P^T (P rounded to bf16).
//  - Online softmax in log2 units with the same lazy rescale as decode.
//  - Workgroups loop over the work list; item % num_kv_heads is the KV head,
//    so with 8 KV heads and a grid that is a multiple of 8 every XCD serves
//    one KV head and re-reads its K/V from its own L2.
#include <algorithm>
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;
constexpr int kWaveTokens = 32;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Tokens per workgroup tile for a given number of heads per workgroup.
constexpr int tile_tokens(int hw) { return kWaveTokens * (kWaves / hw); }

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* qsl, int64_t S, int64_t T, int qtile,
                                                    int32_t* tile_start) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (S + 1023) / 1024;
  const int64_t s0 = min(S, tid * per), s1 = min(S, s0 + per);
  auto tiles = [&](int64_t s) -> int32_t {
    const int64_t a = min(max(static_cast<int64_t>(qsl[s]), int64_t(0)), T);
    const int64_t b = min(max(static_cast<int64_t>(qsl[s + 1]), a), T);
    const int64_t n = b - a;
    return n > 1 ? static_cast<int32_t>((n + qtile - 1) / qtile) : 0;
  };
  int32_t sum = 0;
  for (int64_t s = s0; s < s1; ++s) sum += tiles(s);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
  for (int64_t s = s0; s < s1; ++s) {
    tile_start[s] = run;
    run += tiles(s);
  }
  if (tid == 1023) tile_start[S] = part[1023];
}

template <bool BF16, int D>
struct PrefillShape {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int KT = BF16 ? 64 : 32;     // keys per LDS stage
  static constexpr int KPAD = BF16 ? 8 : 4;     // row padding of K tile (elements)
  static constexpr int VPAD = 4;                // row padding of V^T tile (elements)
  static constexpr int QF = BF16 ? D / 16 : D / 2;  // Q fragments per lane
  using E = typename std::conditional<BF16, uint16_t, float>::type;
};

template <bool BF16, int D, int HW>
__global__ __launch_bounds__(kThreads) void prefill_kernel(AttnArgs a) {
  using Sh = PrefillShape<BF16, D>;
  using E = typename Sh::E;
  constexpr int KT = Sh::KT, ES = Sh::ES;
  constexpr int KROW = D + Sh::KPAD;   // elements per K tile row
  constexpr int VROW = KT + Sh::VPAD;  // elements per V^T tile row
  constexpr int QTB = tile_tokens(HW);
  constexpr int VPR = D * ES / 16;     // 16-byte vectors per K/V row
  __shared__ __attribute__((aligned(16))) E ks[KT * KROW];
  __shared__ __attribute__((aligned(16))) E vt[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 31;  // query token of this lane (B/C column)
  const int hh = lane >> 5;   // lane half
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wave % HW, tw = wave / HW;
  const int G = static_cast<int>(a.Hq / a.Hkv);
  const int n_hg = G / HW;
  const int64_t total_tiles = a.tile_start[a.S];
  const int64_t items = total_tiles * a.Hkv * n_hg;
  const float qk_scale = a.scale * kLog2e;

  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t g = it % a.Hkv;
    const int64_t rest = it / a.Hkv;
    const int64_t hg = rest % n_hg;
    const int64_t trank = rest / n_hg;
    // sequence owning tile `trank`: last s with tile_start[s] <= trank
    int64_t lo = 0, hi = a.S - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (a.tile_start[mid] <= trank) lo = mid; else hi = mid - 1;
    }
    const int64_t s = lo;
    const int64_t ntiles = a.tile_start[s + 1] - a.tile_start[s];
    const int64_t lt = ntiles - 1 - (trank - a.tile_start[s]);  // heavier (later) tiles first
    const int64_t q0 = min(max(static_cast<int64_t>(a.qsl[s]), int64_t(0)), a.T);
    const int64_t n = min(max(static_cast<int64_t>(a.qsl[s + 1]), q0), a.T) - q0;
    const int64_t C = max(static_cast<int64_t>(a.ctx_lens[s]), int64_t(0));
    const int64_t Lc = min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens);
    const int64_t h = g * G + hg * HW + hw;
    const int64_t i0 = lt * QTB + tw * kWaveTokens;  // first token of this wave
    const bool wave_active = i0 < n;
    const int64_t blk_last = min(n, (lt + 1) * QTB) - 1;      // last token of the tile
    const int64_t kend = min(C + blk_last + 1, Lc);           // keys [0, kend) needed by the tile
    const int64_t wave_kend = wave_active ? min(C + min(n, i0 + kWaveTokens), Lc) : 0;
    const int64_t my_i = min(i0 + col, n - 1);                // clamped token of this lane
    const int64_t my_pos = C + my_i;                          // last visible key of this lane

    // Q^T fragments (B operand of S^T = K . Q^T)
    typedef typename std::conditional<BF16, bf16x8, float>::type QFrag;
    QFrag qf[Sh::QF];
    {
      const char* qrow = a.q + (q0 + my_i) * a.q_st + h * a.q_sh;
      if constexpr (BF16) {
#pragma unroll
        for (int st = 0; st < Sh::QF; ++st)
          qf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 2 * (16 * st + 8 * hh)));
      } else {
#pragma unroll
        for (int st = 0; st < Sh::QF; ++st) qf[st] = reinterpret_cast<const float*>(qrow)[2 * st + hh];
      }
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
      // stage K rows [k0, k0 + KT) row-major
      for (int v = tid; v < KT * VPR; v += kThreads) {
        const int key = v / VPR, c = v % VPR;
        const int64_t j = k0 + key;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (j < kend) {
          int64_t id = bt[j / kBlockTokens];
          id = static_cast<uint64_t>(id) < static_cast<uint64_t>(a.NB) ? id : 0;
          val = *reinterpret_cast<const uint4*>(kc + id * a.kc_sb + (j % kBlockTokens) * a.kc_sr + 16 * c);
        }
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(ks) + (key * KROW) * ES + 16 * c) = val;
      }
      // stage V rows transposed: vt[d][key]
      if constexpr (BF16) {
        // pairs of keys -> 32-bit words (V[key][d], V[key + 1][d])
        for (int v = tid; v < (KT / 2) * VPR; v += kThreads) {
          const int kp = v / VPR, c = v % VPR;
          uint4 r0 = make_uint4(0, 0, 0, 0), r1 = make_uint4(0, 0, 0, 0);
          const int64_t j = k0 + 2 * kp;
          if (j < kend) {
            int64_t id = bt[j / kBlockTokens];
            id = static_cast<uint64_t>(id) < static_cast<uint64_t>(a.NB) ? id : 0;
            r0 = *reinterpret_cast<const uint4*>(vc + id * a.vc_sb + (j % kBlockTokens) * a.vc_sr + 16 * c);
          }
          if (j + 1 < kend) {
            int64_t id = bt[(j + 1) / kBlockTokens];
            id = static_cast<uint64_t>(id) < static_cast<uint64_t>(a.NB) ? id : 0;
            r1 = *reinterpret_cast<const uint4*>(vc + id * a.vc_sb + ((j + 1) % kBlockTokens) * a.vc_sr + 16 * c);
          }
          const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
          const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
          uint32_t* base = reinterpret_cast<uint32_t*>(vt);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d = 8 * c + 2 * e;
            base[(d * VROW + 2 * kp) / 2] = (w0[e] & 0xffffu) | (w1[e] << 16);
            base[((d + 1) * VROW + 2 * kp) / 2] = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
          }
        }
      } else {
        for (int v = tid; v < KT * VPR; v += kThreads) {
          const int key = v / VPR, c = v % VPR;
          const int64_t j = k0 + key;
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (j < kend) {
            int64_t id = bt[j / kBlockTokens];
            id = static_cast<uint64_t>(id) < static_cast<uint64_t>(a.NB) ? id : 0;
            f = *reinterpret_cast<const float4*>(vc + id * a.vc_sb + (j % kBlockTokens) * a.vc_sr + 16 * c);
          }
          float* base = reinterpret_cast<float*>(vt);
          base[(4 * c + 0) * VROW + key] = f.x;
          base[(4 * c + 1) * VROW + key] = f.y;
          base[(4 * c + 2) * VROW + key] = f.z;
          base[(4 * c + 3) * VROW + key] = f.w;
        }
      }
      __syncthreads();
      if (!wave_active) continue;

#pragma unroll
      for (int half = 0; half < KT / 32; ++half) {
        const int64_t kh0 = k0 + 32 * half;
        if (kh0 >= wave_kend) break;
        // S^T[key kh0 + 8q + 4hh + r][token col] in sacc[4q + r]
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
        if constexpr (BF16) {
#pragma unroll
          for (int st = 0; st < Sh::QF; ++st) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&ks[(32 * half + col) * KROW + 16 * st + 8 * hh]);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], sacc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int st = 0; st < Sh::QF; ++st) {
            const float kf = ks[(32 * half + col) * KROW + 2 * st + hh];
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf, qf[st], sacc, 0, 0, 0);
          }
        }
        float sc[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = kh0 + 8 * (i >> 2) + 4 * hh + (i & 3);
          sc[i] = (key <= my_pos && key < kend) ? sacc[i] * qk_scale : -INFINITY;
          tmax = fmaxf(tmax, sc[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        if (__any(tmax > m_run + kRescaleThreshold)) {
          const float m_new = fmaxf(m_run, tmax);
          const float alpha = fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
          m_run = m_new;
        }
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pv[i] = fast_exp2(sc[i] - m_run);
          l_run += pv[i];
        }
        // O^T[d][token] += V^T[d][key] P^T[key][token]
        if constexpr (BF16) {
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(pv[8 * q2 + e]);
            // key slots: e < 4 -> 16 q2 + 4 hh + e; e >= 4 -> 16 q2 + 8 + 4 hh + (e - 4)
            const int kb = 32 * half + 16 * q2 + 4 * hh;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
              const E* row = &vt[(32 * dt + col) * VROW];
              const uint2 lo = *reinterpret_cast<const uint2*>(row + kb);
              const uint2 hi = *reinterpret_cast<const uint2*>(row + kb + 8);
              const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * half + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
              const float va = vt[(32 * dt + col) * VROW + key];
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, pv[i], o[dt], 0, 0, 0);
            }
          }
        }
      }
    }

    if (wave_active) {
      float l_tot = l_run + __shfl_xor(l_run, 32);
      const int64_t my_tok = i0 + col;
      if (my_tok < n) {
        const float inv = 1.f / l_tot;
        char* dst = a.out + (q0 + my_tok) * a.out_st + h * a.out_sh;
        // lane holds O^T[d = 32 dt + 8 q + 4 hh + r][token col]
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int d = 32 * dt + 8 * q + 4 * hh;
            if constexpr (BF16) {
              *reinterpret_cast<uint2*>(dst + 2 * d) =
                  make_uint2(pack_bf16(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv),
                             pack_bf16(o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv));
            } else {
              *reinterpret_cast<float4*>(dst + 4 * d) =
                  make_float4(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv, o[dt][4 * q + 2] * inv,
                              o[dt][4 * q + 3] * inv);
            }
          }
      }
    }
  }
}

template <bool BF16, int D, int HW>
hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
  constexpr int QTB = tile_tokens(HW);
  {
    ProfileScope ps(kPlan, stream);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.qsl, a.S, a.T, QTB, a.tile_start);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Upper bound on tiles without reading lengths: every prefill sequence has
  // at least two tokens.
  const int64_t tiles_ub = a.T / QTB + std::min<int64_t>(a.S, a.T / 2);
  const int64_t G = a.Hq / a.Hkv;
  const int64_t items_ub = tiles_ub * a.Hkv * (G / HW);
  if (items_ub == 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>((items_ub + 7) / 8 * 8, 2048);
  {
    ProfileScope ps(kPrefill, stream);
    hipLaunchKernelGGL((prefill_kernel<BF16, D, HW>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                       a);
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

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  const bool bf16 = a.elem == Elem::BF16;
  if (a.D == 64) return bf16 ? launch_heads<true, 64>(a, stream) : launch_heads<false, 64>(a, stream);
  return bf16 ? launch_heads<true, 128>(a, stream) : launch_heads<false, 128>(a, stream);
}

}  // namespace pa
