// KV write: scatter each new token's K and V rows into its slot of the block
// pool. Slot s names block s / 16, row s % 16 ("Inside vLLM", section "Run
// forward pass", step 2 builds slot_mapping; the forward pass then fills the
// paged KV cache). A bitwise copy in 16-byte vectors; HBM-bound.
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

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
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
