// Device pieces shared by the kernels of more than one source file:
//  - the KV write of one workgroup's tokens (kv_write.hip's kernels, and the
//    plan kernel's launch that also writes, prefill.hip);
//  - the combination of a sequence's split-K partitions for one query head
//    (decode.hip's reduce kernel, and the prefill kernel when it runs after
//    the decode on the same stream).
#pragma once

#include "pa_internal.h"

namespace pa {

__device__ inline uint32_t pack2_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// KV write of tokens [block * tpb, block * tpb + tpb) by the workgroup's
// nthreads lanes: the lanes walk the 16-byte vectors of those tokens' K rows,
// then V rows, so that neighbouring lanes read neighbouring bytes of k/v and
// write neighbouring bytes of one pool row. Negative or past-the-pool slots
// are skipped.
__device__ inline void kv_write_tokens(const WriteArgs& a, int vec_per_head, int tpb, int64_t block, int nthreads) {
  const int vec_per_row = static_cast<int>(a.Hkv) * vec_per_head;  // one K (or V) row
  const int vec_per_tok = 2 * vec_per_row;
  const int64_t t0 = block * tpb;
  const uint64_t nslots = static_cast<uint64_t>(a.NB) * kBlockTokens;
  for (int i = threadIdx.x; i < tpb * vec_per_tok; i += nthreads) {
    const int tl = i / vec_per_tok;
    const int64_t t = t0 + tl;
    if (t >= a.T) break;
    int r = i - tl * vec_per_tok;
    const bool is_v = r >= vec_per_row;
    r -= is_v ? vec_per_row : 0;
    const int h = r / vec_per_head;
    const int c = r - h * vec_per_head;
    const int64_t slot = a.slots[t];
    if (static_cast<uint64_t>(slot) >= nslots) continue;  // negative (padding) or past the pool
    const int64_t blk = slot >> 4, row = slot & 15;
    const char* src = is_v ? a.v + t * a.v_st + h * a.v_sh : a.k + t * a.k_st + h * a.k_sh;
    char* dst = is_v ? a.vc + blk * a.vc_sb + row * a.vc_sr + h * a.vc_sh
                     : a.kc + blk * a.kc_sb + row * a.kc_sr + h * a.kc_sh;
    const uint4 val = *reinterpret_cast<const uint4*>(src + c * 16);
    *reinterpret_cast<uint4*>(dst + c * 16) = val;
  }}

// Nearest OCP FP8 E4M3 code to x: ties to the even code, magnitudes from
// 464 up (past the midpoint above 448) saturate to 448, NaN gives 0x7F; the
// sign is x's sign bit. Works on x's fp32 bits: 2^-6 .. 448 are normal codes
// (4 exponent bits, bias 7; the 20 dropped mantissa bits are rounded), and
// below 2^-6 a code is the count of 2^-9 steps, rounded.
__device__ inline uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;       // NaN
  if (a >= 0x43e80000u) return sign | 0x7eu;      // >= 464 (and inf): saturate
  if (a < 0x3c800000u) {                          // < 2^-6: steps of 2^-9
    const float t = __uint_as_float(a) * 512.0f;  // exact: a power-of-two scaling
    return sign | static_cast<uint32_t>(__builtin_rintf(t));  // nearest, ties to even; 8 is 2^-6 (code 8)
  }
  uint32_t keep = (a >> 20) & 7u;
  const uint32_t rest = a & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;  // carry into the exponent is exact
  return sign | ((((a >> 23) - 120u) << 3) + keep);
}

// KV write into an fp8 pool: like kv_write_tokens, but a vector is 16 output
// codes (16 elements of k or v), each nearest(x / scale).
__device__ inline void kv_write_fp8_tokens(const WriteArgs& a, int vec_per_head, int tpb, int64_t block,
                                           int nthreads) {
  const int vec_per_row = static_cast<int>(a.Hkv) * vec_per_head;
  const int vec_per_tok = 2 * vec_per_row;
  const int64_t t0 = block * tpb;
  const uint64_t nslots = static_cast<uint64_t>(a.NB) * kBlockTokens;
  for (int i = threadIdx.x; i < tpb * vec_per_tok; i += nthreads) {
    const int tl = i / vec_per_tok;
    const int64_t t = t0 + tl;
    if (t >= a.T) break;
    int r = i - tl * vec_per_tok;
    const bool is_v = r >= vec_per_row;
    r -= is_v ? vec_per_row : 0;
    const int h = r / vec_per_head;
    const int c = r - h * vec_per_head;
    const int64_t slot = a.slots[t];
    if (static_cast<uint64_t>(slot) >= nslots) continue;
    const int64_t blk = slot >> 4, row = slot & 15;
    const char* src = is_v ? a.v + t * a.v_st + h * a.v_sh : a.k + t * a.k_st + h * a.k_sh;
    char* dst = is_v ? a.vc + blk * a.vc_sb + row * a.vc_sr + h * a.vc_sh
                     : a.kc + blk * a.kc_sb + row * a.kc_sr + h * a.kc_sh;
    const float sc = is_v ? a.v_scale : a.k_scale;
    float x[16];
    if (a.es == 2) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(src + c * 32 + 16 * q);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * q + 2 * e] = __uint_as_float(ws[e] << 16);
          x[8 * q + 2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(src + c * 64 + 16 * q);
        x[4 * q] = f.x;
        x[4 * q + 1] = f.y;
        x[4 * q + 2] = f.z;
        x[4 * q + 3] = f.w;
      }
    }
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[q] |= e4m3_code(x[4 * q + e] / sc) << (8 * e);
    }
    *reinterpret_cast<uint4*>(dst + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Combine the split-K partitions of decode-kernel sequence s = item / Hq for
// query head item % Hq, for each of its new tokens, in fixed partition order,
// by one wave (lane = this lane); a no-op for other items.
template <bool BF16, int D>
__device__ inline void reduce_partitions(const AttnArgs& a, int64_t item, int lane) {
  constexpr int DPL = D / 64;  // output elements per lane
  const int64_t s = item / a.Hq, hq = item - s * a.Hq;
  if (s >= a.S) return;
  const int q0 = a.qsl[s], q1 = a.qsl[s + 1];
  if (!decode_path(q1 - q0, a.Hq / a.Hkv) || q0 < 0 || q1 > a.T) return;
  const int64_t L = min(max(static_cast<int64_t>(a.seq_lens[s]), int64_t(0)), a.MB * kBlockTokens);
  const int nparts = static_cast<int>((L + a.part_tokens - 1) / a.part_tokens);
  if (nparts <= 1) return;
  for (int64_t t = q0; t < q1; ++t) {
    const float2* ml = a.ws_ml + (t * a.Hq + hq) * a.max_parts;
    const float* po = a.ws_o + (t * a.Hq + hq) * a.max_parts * D + DPL * lane;
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
        w = __builtin_amdgcn_exp2f(v.x - m);
        lsum += w * v.y;
      }
      const int cnt = min(64, nparts - p0);
      // eight partitions' values are loaded before any is used, so their
      // loads are in flight together
      for (int j0 = 0; j0 < cnt; j0 += 8) {
        float x[8][DPL];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float* src = po + int64_t(p0 + min(j0 + j, cnt - 1)) * D;
          if constexpr (DPL == 2) {
            const float2 v = *reinterpret_cast<const float2*>(src);
            x[j][0] = v.x;
            x[j][1] = v.y;
          } else {
            x[j][0] = src[0];
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float wj = j0 + j < cnt ? __shfl(w, j0 + j) : 0.f;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] += wj * x[j][e];
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
    const float inv = 1.f / lsum;
    char* dst = a.out + t * a.out_st + hq * a.out_sh;
    if constexpr (BF16) {
      if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(dst + 4 * lane) = pack2_bf16(acc[0] * inv, acc[1] * inv);
      } else {
        reinterpret_cast<__bf16*>(dst)[lane] = static_cast<__bf16>(acc[0] * inv);
      }
    } else {
#pragma unroll
      for (int i = 0; i < DPL; ++i) reinterpret_cast<float*>(dst)[DPL * lane + i] = acc[i] * inv;
    }
  }
}

}  // namespace pa
