// KV write: scatter each new token's K and V rows into its slot of the block
// pool. Slot s names block s / 16, row s % 16 ("Inside vLLM", section "Run
// forward pass", step 2 builds slot_mapping; the forward pass then fills the
// paged KV cache). A bitwise copy in 16-byte vectors; HBM-bound. An 8-bit
// pool stores each element's nearest OCP FP8 E4M3 code of x / scale instead.
//
// Work layout: one workgroup owns `tpb` consecutive tokens; its 256 lanes
// walk the 16-byte vectors of those tokens' K rows then V rows, so lanes that
// are neighbours read neighbouring bytes of k/v and write neighbouring bytes
// of one pool row.
#include "pa_internal.h"

namespace pa {
namespace {

__global__ __launch_bounds__(kThreads) void kv_write_kernel(WriteArgs a, int vec_per_head, int tpb) {
  const int vec_per_row = static_cast<int>(a.Hkv) * vec_per_head;  // one K (or V) row
  const int vec_per_tok = 2 * vec_per_row;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
  const uint64_t nslots = static_cast<uint64_t>(a.NB) * kBlockTokens;
  for (int i = threadIdx.x; i < tpb * vec_per_tok; i += kThreads) {
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
  }
}

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

// KV write into an fp8 pool: like kv_write_kernel, but a vector is 16 output
// codes (16 elements of k or v), each nearest(x / scale).
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(WriteArgs a, int vec_per_head, int tpb) {
  const int vec_per_row = static_cast<int>(a.Hkv) * vec_per_head;
  const int vec_per_tok = 2 * vec_per_row;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
  const uint64_t nslots = static_cast<uint64_t>(a.NB) * kBlockTokens;
  for (int i = threadIdx.x; i < tpb * vec_per_tok; i += kThreads) {
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

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  if (a.kv8) {
    const int vec_per_head = static_cast<int>(a.D / 16);  // 16 codes per vector
    const int vec_per_tok = 2 * static_cast<int>(a.Hkv) * vec_per_head;
    const int tpb = vec_per_tok >= kThreads ? 1 : kThreads / vec_per_tok;
    const int64_t blocks = (a.T + tpb - 1) / tpb;
    ProfileScope ps(kKvWrite, stream);
    hipLaunchKernelGGL(kv_write_fp8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, a,
                       vec_per_head, tpb);
    return hipGetLastError();
  }
  const int vec_per_head = static_cast<int>(a.D * a.es / 16);
  const int vec_per_tok = 2 * static_cast<int>(a.Hkv) * vec_per_head;
  // Enough tokens per workgroup that every lane has at least one vector.
  const int tpb = vec_per_tok >= kThreads ? 1 : kThreads / vec_per_tok;
  const int64_t blocks = (a.T + tpb - 1) / tpb;
  {
    ProfileScope ps(kKvWrite, stream);
    hipLaunchKernelGGL(kv_write_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, a,
                       vec_per_head, tpb);
  }
  return hipGetLastError();
}

}  // namespace pa
