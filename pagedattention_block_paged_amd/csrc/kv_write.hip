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
#include "step_parts.h"

namespace pa {
namespace {

__global__ __launch_bounds__(kThreads) void kv_write_kernel(WriteArgs a, int vec_per_head, int tpb) {
  kv_write_tokens(a, vec_per_head, tpb, blockIdx.x, kThreads);
}

__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(WriteArgs a, int vec_per_head, int tpb) {
  kv_write_fp8_tokens(a, vec_per_head, tpb, blockIdx.x, kThreads);
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
