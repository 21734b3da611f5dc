// C-ABI entry points of libpa.so: host-side validation of the tensor
// descriptors, workspace layout, and dispatch to the HIP kernel launchers.
// The descriptor checks touch no device memory and do not synchronise, so
// they run (and are tested) on a machine without a GPU. Only the opt-in
// content check (environment PA_VALIDATE=1) copies the metadata to the host.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace

namespace pa {

pa_status report(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status report_ok() { return ok(); }

}  // namespace pa

namespace {

int64_t elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_I32: return 4;
    case PA_I64: return 8;
    case PA_FP8_E4M3: return 1;
    default: return 0;
  }
}

const char* dtype_name(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return "f32";
    case PA_BF16: return "bf16";
    case PA_I32: return "i32";
    case PA_I64: return "i64";
    case PA_FP8_E4M3: return "fp8_e4m3";
    default: return "?";
  }
}

int64_t numel(const pa_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// Descriptor sanity: present, rank, dtype, non-negative extents, data present
// unless empty.
pa_status check_desc(const pa_tensor* t, const char* name, int ndim) {
  if (!t) return fail(PA_ERR_NULL, "%s: descriptor is NULL", name);
  if (t->ndim != ndim) return fail(PA_ERR_SHAPE, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  if (elem_bytes(t->dtype) == 0) return fail(PA_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(PA_ERR_SHAPE, "%s: negative extent in dim %d", name, i);
  if (!t->data && numel(t) > 0) return fail(PA_ERR_NULL, "%s: data pointer is NULL", name);
  return PA_OK;
}

pa_status check_dtype(const pa_tensor* t, const char* name, int32_t want) {
  if (t->dtype != want)
    return fail(PA_ERR_DTYPE, "%s: dtype %s, expected %s", name, dtype_name(t->dtype), dtype_name(want));
  return PA_OK;
}

// A float tensor whose last dim is contiguous and whose rows are 16-byte
// aligned (the kernels move rows in 16-byte vectors).
pa_status check_rows(const pa_tensor* t, const char* name) {
  if (t->stride[t->ndim - 1] != 1 && t->shape[t->ndim - 1] > 1)
    return fail(PA_ERR_STRIDE, "%s: last dim must be contiguous (stride %lld)", name,
                (long long)t->stride[t->ndim - 1]);
  const int64_t es = elem_bytes(t->dtype);
  if (reinterpret_cast<uintptr_t>(t->data) % 16)
    return fail(PA_ERR_STRIDE, "%s: data pointer not 16-byte aligned", name);
  for (int i = 0; i + 1 < t->ndim; ++i)
    if ((t->stride[i] * es) % 16 || t->stride[i] < 0)
      return fail(PA_ERR_STRIDE, "%s: stride of dim %d (%lld elements) is not a multiple of 16 bytes", name, i,
                  (long long)t->stride[i]);
  return PA_OK;
}

pa_status check_contig1(const pa_tensor* t, const char* name) {
  if (t->shape[0] > 1 && t->stride[0] != 1) return fail(PA_ERR_STRIDE, "%s: must be contiguous", name);
  return PA_OK;
}

#define PA_TRY(expr)                  \
  do {                                \
    pa_status _st = (expr);           \
    if (_st != PA_OK) return _st;     \
  } while (0)

struct CacheShape {
  int64_t NB, Hkv, D;
  int32_t dtype;
};

pa_status check_caches(const pa_tensor* kc, const pa_tensor* vc, bool fp8, CacheShape* cs) {
  PA_TRY(check_desc(kc, "key_cache", 4));
  PA_TRY(check_desc(vc, "value_cache", 4));
  if (fp8 && kc->dtype != PA_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "key_cache: dtype %s, expected fp8_e4m3", dtype_name(kc->dtype));
  if (!fp8 && kc->dtype == PA_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "key_cache: fp8_e4m3 caches go through the _fp8 calls (they take the scales)");
  if (!fp8 && kc->dtype != PA_F32 && kc->dtype != PA_BF16)
    return fail(PA_ERR_DTYPE, "key_cache: dtype %s, expected f32 or bf16", dtype_name(kc->dtype));
  PA_TRY(check_dtype(vc, "value_cache", kc->dtype));
  for (int i = 0; i < 4; ++i)
    if (kc->shape[i] != vc->shape[i]) return fail(PA_ERR_SHAPE, "key_cache and value_cache shapes differ (dim %d)", i);
  if (kc->shape[1] != pa::kBlockTokens)
    return fail(PA_ERR_UNSUPPORTED, "block size %lld not supported (only 16)", (long long)kc->shape[1]);
  if (kc->shape[0] < 1) return fail(PA_ERR_SHAPE, "key_cache: pool has no blocks");
  PA_TRY(check_rows(kc, "key_cache"));
  PA_TRY(check_rows(vc, "value_cache"));
  cs->NB = kc->shape[0];
  cs->Hkv = kc->shape[2];
  cs->D = kc->shape[3];
  cs->dtype = kc->dtype;
  if (cs->Hkv < 1 || cs->D < 1) return fail(PA_ERR_SHAPE, "key_cache: empty head dims");
  if ((cs->D * elem_bytes(cs->dtype)) % 16)
    return fail(PA_ERR_UNSUPPORTED, "head_size %lld: cache rows must be a multiple of 16 bytes", (long long)cs->D);
  return PA_OK;
}

pa_status check_scales(float k_scale, float v_scale) {
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must be finite and > 0 (got %g, %g)", k_scale, v_scale);
  return PA_OK;
}

pa_status validate_write(const pa_tensor* k, const pa_tensor* v, const pa_tensor* kc, const pa_tensor* vc,
                         const pa_tensor* slots, bool fp8, float k_scale, float v_scale, pa::WriteArgs* a) {
  CacheShape cs;
  PA_TRY(check_caches(kc, vc, fp8, &cs));
  PA_TRY(check_desc(k, "k", 3));
  PA_TRY(check_desc(v, "v", 3));
  PA_TRY(check_desc(slots, "slot_mapping", 1));
  if (fp8) {
    PA_TRY(check_scales(k_scale, v_scale));
    if (k->dtype != PA_F32 && k->dtype != PA_BF16)
      return fail(PA_ERR_DTYPE, "k: dtype %s, expected f32 or bf16", dtype_name(k->dtype));
    PA_TRY(check_dtype(v, "v", k->dtype));
  } else {
    PA_TRY(check_dtype(k, "k", cs.dtype));
    PA_TRY(check_dtype(v, "v", cs.dtype));
  }
  PA_TRY(check_dtype(slots, "slot_mapping", PA_I64));
  const int64_t T = k->shape[0];
  for (int i = 0; i < 3; ++i)
    if (k->shape[i] != v->shape[i]) return fail(PA_ERR_SHAPE, "k and v shapes differ (dim %d)", i);
  if (k->shape[1] != cs.Hkv || k->shape[2] != cs.D)
    return fail(PA_ERR_SHAPE, "k is [%lld, %lld, %lld], cache heads/dims are [%lld, %lld]", (long long)T,
                (long long)k->shape[1], (long long)k->shape[2], (long long)cs.Hkv, (long long)cs.D);
  if (slots->shape[0] != T)
    return fail(PA_ERR_SHAPE, "slot_mapping has %lld entries for %lld tokens", (long long)slots->shape[0],
                (long long)T);
  const int64_t es = elem_bytes(k->dtype), ces = elem_bytes(cs.dtype);
  if ((cs.D * es) % 16) return fail(PA_ERR_UNSUPPORTED, "head_size %lld: rows must be a multiple of 16 bytes",
                                    (long long)cs.D);
  PA_TRY(check_contig1(slots, "slot_mapping"));
  if (T > 0) {
    PA_TRY(check_rows(k, "k"));
    PA_TRY(check_rows(v, "v"));
  }
  a->k = static_cast<const char*>(k->data);
  a->v = static_cast<const char*>(v->data);
  a->kc = static_cast<char*>(kc->data);
  a->vc = static_cast<char*>(vc->data);
  a->slots = static_cast<const int64_t*>(slots->data);
  a->T = T;
  a->Hkv = cs.Hkv;
  a->D = cs.D;
  a->NB = cs.NB;
  a->k_st = k->stride[0] * es;
  a->k_sh = k->stride[1] * es;
  a->v_st = v->stride[0] * es;
  a->v_sh = v->stride[1] * es;
  a->kc_sb = kc->stride[0] * ces;
  a->kc_sr = kc->stride[1] * ces;
  a->kc_sh = kc->stride[2] * ces;
  a->vc_sb = vc->stride[0] * ces;
  a->vc_sr = vc->stride[1] * ces;
  a->vc_sh = vc->stride[2] * ces;
  a->es = static_cast<int>(es);
  a->kv8 = fp8;
  a->k_scale = k_scale;
  a->v_scale = v_scale;
  return PA_OK;
}

pa_status validate_attention(const pa_tensor* out, const pa_tensor* q, const pa_tensor* kc, const pa_tensor* vc,
                             const pa_tensor* bt, const pa_tensor* qsl, const pa_tensor* sl, const pa_tensor* cl,
                             float scale, bool fp8, float k_scale, float v_scale, void* ws, size_t ws_bytes,
                             pa::AttnArgs* a) {
  CacheShape cs;
  PA_TRY(check_caches(kc, vc, fp8, &cs));
  if (fp8) PA_TRY(check_scales(k_scale, v_scale));
  const int32_t qdt = fp8 ? PA_BF16 : cs.dtype;  // fp8 caches compute in bf16
  PA_TRY(check_desc(out, "out", 3));
  PA_TRY(check_desc(q, "q", 3));
  PA_TRY(check_desc(bt, "block_tables", 2));
  PA_TRY(check_desc(qsl, "query_start_loc", 1));
  PA_TRY(check_desc(sl, "seq_lens", 1));
  PA_TRY(check_desc(cl, "context_lens", 1));
  PA_TRY(check_dtype(q, "q", qdt));
  PA_TRY(check_dtype(out, "out", qdt));
  PA_TRY(check_dtype(bt, "block_tables", PA_I32));
  PA_TRY(check_dtype(qsl, "query_start_loc", PA_I32));
  PA_TRY(check_dtype(sl, "seq_lens", PA_I32));
  PA_TRY(check_dtype(cl, "context_lens", PA_I32));
  const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PA_ERR_SHAPE, "out and q shapes differ (dim %d)", i);
  if (D != cs.D) return fail(PA_ERR_SHAPE, "q head_size %lld != cache head_size %lld", (long long)D, (long long)cs.D);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "head_size %lld not supported (64 or 128)", (long long)D);
  if (Hq < 1 || Hq % cs.Hkv)
    return fail(PA_ERR_SHAPE, "num_q_heads %lld is not a multiple of num_kv_heads %lld", (long long)Hq,
                (long long)cs.Hkv);
  if (Hq / cs.Hkv > 16)
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head %lld > 16", (long long)(Hq / cs.Hkv));
  const int64_t S = bt->shape[0], MB = bt->shape[1];
  if (MB < 1) return fail(PA_ERR_SHAPE, "block_tables has no columns");
  if (qsl->shape[0] != S + 1)
    return fail(PA_ERR_SHAPE, "query_start_loc has %lld entries for %lld sequences", (long long)qsl->shape[0],
                (long long)S);
  if (sl->shape[0] != S || cl->shape[0] != S) return fail(PA_ERR_SHAPE, "seq_lens/context_lens must have S entries");
  if (bt->stride[1] != 1 && MB > 1) return fail(PA_ERR_STRIDE, "block_tables rows must be contiguous");
  if (bt->stride[0] < MB && S > 1) return fail(PA_ERR_STRIDE, "block_tables rows overlap");
  PA_TRY(check_contig1(qsl, "query_start_loc"));
  PA_TRY(check_contig1(sl, "seq_lens"));
  PA_TRY(check_contig1(cl, "context_lens"));
  if (T > 0) {
    PA_TRY(check_rows(q, "q"));
    PA_TRY(check_rows(out, "out"));
  }
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "scale is not finite");
  const pa::WorkspaceLayout wl = pa::workspace_layout(S, T, Hq, cs.Hkv, D, MB);
  if (ws_bytes < wl.total)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, wl.total);
  if (wl.total > 0 && !ws) return fail(PA_ERR_WORKSPACE, "workspace pointer is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(PA_ERR_WORKSPACE, "workspace not 256-byte aligned");

  const int64_t es = elem_bytes(qdt), ces = elem_bytes(cs.dtype);
  a->out = static_cast<char*>(out->data);
  a->q = static_cast<const char*>(q->data);
  a->kc = static_cast<const char*>(kc->data);
  a->vc = static_cast<const char*>(vc->data);
  a->block_tables = static_cast<const int32_t*>(bt->data);
  a->qsl = static_cast<const int32_t*>(qsl->data);
  a->seq_lens = static_cast<const int32_t*>(sl->data);
  a->ctx_lens = static_cast<const int32_t*>(cl->data);
  a->T = T;
  a->S = S;
  a->MB = MB;
  a->NB = cs.NB;
  a->Hq = Hq;
  a->Hkv = cs.Hkv;
  a->D = D;
  a->out_st = out->stride[0] * es;
  a->out_sh = out->stride[1] * es;
  a->q_st = q->stride[0] * es;
  a->q_sh = q->stride[1] * es;
  a->kc_sb = kc->stride[0] * ces;
  a->kc_sr = kc->stride[1] * ces;
  a->kc_sh = kc->stride[2] * ces;
  a->vc_sb = vc->stride[0] * ces;
  a->vc_sr = vc->stride[1] * ces;
  a->vc_sh = vc->stride[2] * ces;
  a->bt_row = S > 1 ? bt->stride[0] : MB;
  a->scale = scale;
  a->elem = qdt == PA_F32 ? pa::Elem::F32 : pa::Elem::BF16;
  a->kv8 = fp8;
  a->k_scale = fp8 ? k_scale : 1.f;
  a->v_scale = fp8 ? v_scale : 1.f;
  a->part_tokens = pa::partition_tokens(S, cs.Hkv, MB, pa::decode_workgroups_per_cu(a->elem, a->kv8, D));
  a->max_parts = (MB * pa::kBlockTokens + a->part_tokens - 1) / a->part_tokens;
  if (MB > (int64_t(1) << 26) || a->max_parts > 65535)
    return fail(PA_ERR_UNSUPPORTED, "block_tables has too many columns (%lld)", (long long)MB);
  if (S * cs.Hkv > int64_t(0x7fffffff)) return fail(PA_ERR_UNSUPPORTED, "too many sequences x KV heads");
  // In-block byte offsets (row within a block, head slice) are 32-bit in the kernels.
  if (std::max(a->kc_sr, a->vc_sr) * pa::kBlockTokens + D * ces > int64_t(0x7fffffff))
    return fail(PA_ERR_UNSUPPORTED, "cache row stride too large (%lld bytes)", (long long)std::max(a->kc_sr, a->vc_sr));
  char* base = static_cast<char*>(ws);
  a->tile_start = reinterpret_cast<int32_t*>(base + wl.tile_start_off);
  a->work_counter = reinterpret_cast<int32_t*>(base + wl.counter_off);
  a->tile_order = reinterpret_cast<int32_t*>(base + wl.order_off);
  a->sched = reinterpret_cast<int32_t*>(base + wl.sched_off);
  a->dorder = reinterpret_cast<int32_t*>(base + wl.dorder_off);
  a->ws_ml = reinterpret_cast<float2*>(base + wl.ml_off);
  a->ws_o = reinterpret_cast<float*>(base + wl.o_off);
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A stream of the library's own and two events per (host thread, device),
// for running the chunked prefill beside the decode kernel. Created on first
// use and kept until the process ends (never destroyed: the runtime may be
// gone by the time thread-local destructors run).
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};

SideStream* side_stream_for(hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static thread_local SideStream side[kMaxDevices];
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& ss = side[dev];
  if (ss.failed) return nullptr;
  if (!ss.stream) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess || (cur != dev && hipSetDevice(dev) != hipSuccess)) {
      ss.failed = true;
      return nullptr;
    }
    // default priority, no implicit synchronisation with the null stream
    const bool ok = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) == hipSuccess &&
                    hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess &&
                    hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
    if (cur != dev) (void)hipSetDevice(cur);
    if (!ok) {
      ss.failed = true;
      return nullptr;
    }
  }
  return &ss;
}

// K/V bytes the decode could read at most: every sequence at the table's full
// width. Above this the decode kernel runs long enough that running the
// prefill beside it pays for the cross-stream hand-off (a few microseconds).
constexpr double kBesideMinDecodeBytes = 4e9;
// The prefill's share of the work, both at the table's full width: every
// query token past one per sequence against every key at the bf16 prefill
// kernel's rate, against every sequence's keys at the decode's HBM rate.
// Below this, running the prefill after the decode on the whole GPU costs
// less than sharing the GPU: on the Llama-3-8B decode batch (4,096 sequences
// of up to 8,192 tokens) with 8 chunks of 512 tokens (2% here) the step took
// 10.64 ms after against 10.74 ms beside; with 64 chunks (17%) 11.76 against
// 11.06 ms, with 160 (42%) 13.57 against 12.42 ms.
constexpr double kBesideMinPrefillShare = 0.05;

// Whether the prefill runs beside the decode: bf16 queries over a bf16 pool,
// a decode that may be long, at least one sequence's worth of tokens past
// one per sequence (a sequence on the prefill path has more than 16 / G new
// tokens; batches of single-token decodes never qualify), and a prefill
// share of at least kBesideMinPrefillShare.
bool prefill_beside_decode(const pa::AttnArgs& a) {
  // bf16 pools only: the prefill of an 8-bit pool widens each tile through
  // registers, and beside the decode's HBM stream it ran 2.5-3x slower than
  // alone, past the decode's end; after the decode it takes about 0.3 ms.
  if (a.elem != pa::Elem::BF16 || a.kv8 || a.S <= 0) return false;
  const int64_t G = a.Hq / a.Hkv;
  if (a.T - a.S < pa::kMaxDecodeColumns / G + 1) return false;
  const double keys = double(a.MB) * pa::kBlockTokens;
  const double decode_bytes = double(a.S) * keys * 2.0 * double(a.Hkv) * double(a.D) * 2.0;
  const double decode_work = decode_bytes / pa::kDecodeBytePerCuUs;
  const double prefill_work = double(a.T - a.S) * keys * 4.0 * double(a.Hq) * double(a.D) / pa::kPrefillFlopPerCuUs;
  return decode_bytes >= kBesideMinDecodeBytes && prefill_work >= kBesideMinPrefillShare * decode_work;
}

// The decode kernel (HBM-bound) and the chunked prefill (MFMA-bound) work on
// disjoint rows of `out` and read only the inputs. For large bf16 batches
// with a large enough prefill (prefill_beside_decode) the prefill runs on a
// second stream, forked from and joined back into
// `stream`, on a few CUs chosen by the plan kernel while the decode streams
// on the rest. Otherwise everything runs on `stream`: the plan (unless the
// caller's KV write launch already made it), the decode, then the prefill
// kernel, which first combines the decode's split-K partitions (one launch
// fewer than a separate reduce).
bool attention_beside(const pa::AttnArgs& a, bool allow_side) {
  return allow_side && a.S > 0 && a.T > 0 && prefill_beside_decode(a);
}

pa_status run_attention(const pa::AttnArgs& a, hipStream_t stream, bool allow_side = true, bool planned = false) {
  if (a.S == 0 || a.T == 0) return PA_OK;
  SideStream* side = attention_beside(a, allow_side) ? side_stream_for(stream) : nullptr;
  if (!side) {
    if (!planned) PA_TRY(hip_status(pa::launch_plan(a, stream, false), "plan launch"));
    const bool fold = a.max_parts > 1 && pa::prefill_launches(a);
    PA_TRY(hip_status(pa::launch_decode(a, stream, !fold), "decode launch"));
    PA_TRY(hip_status(pa::launch_prefill(a, stream, false, fold), "prefill launch"));
    return PA_OK;
  }
  PA_TRY(hip_status(hipEventRecord(side->fork, stream), "fork event"));
  PA_TRY(hip_status(hipStreamWaitEvent(side->stream, side->fork, 0), "fork wait"));
  // plan and prefill first, so that their workgroups take CUs before the decode's
  PA_TRY(hip_status(pa::launch_plan(a, side->stream, true), "plan launch"));
  PA_TRY(hip_status(pa::launch_prefill(a, side->stream, true, false), "prefill launch"));
  PA_TRY(hip_status(pa::launch_decode(a, stream, true), "decode launch"));
  PA_TRY(hip_status(hipEventRecord(side->join, side->stream), "join event"));
  PA_TRY(hip_status(hipStreamWaitEvent(stream, side->join, 0), "join wait"));
  return PA_OK;
}

}  // namespace

namespace pa {

int64_t partition_tokens(int64_t S, int64_t Hkv, int64_t MB, int per_cu) {
  static const int64_t forced = [] {
    const char* e = std::getenv("PA_PARTITION_TOKENS");
    if (!e) return int64_t(0);
    long long v = std::atoll(e);
    return (v >= kBlockTokens && v <= kMaxPartitionTokens && v % kBlockTokens == 0) ? int64_t(v) : int64_t(0);
  }();
  if (forced) return forced;
  // A partition is one decode workgroup's share of a sequence: 8 waves over
  // a group of KV heads. Take the largest partition (fewest partial results)
  // that still yields one round of workgroups on the longest sequences the
  // block table allows: 256 CUs times the workgroups a CU holds at once (one
  // for the bf16 kernel at head size 128, two for the others). A second
  // round of equally long workgroups only adds a tail. At most two per CU
  // count (the workspace is sized for that), and two when unknown.
  const int64_t kMinDecodeWorkgroups = 256 * (per_cu == 1 ? 1 : 2);
  const int64_t groups = S * (Hkv / decode_heads_per_workgroup(Hkv));
  const int64_t max_len = MB * kBlockTokens;
  for (int64_t pt : {kMaxPartitionTokens, int64_t(2048), int64_t(1024), int64_t(512), int64_t(256), int64_t(128),
                     int64_t(64)}) {
    const int64_t parts = (max_len + pt - 1) / pt;
    if (groups * parts >= kMinDecodeWorkgroups) return pt;
  }
  return 64;
}

WorkspaceLayout workspace_layout(int64_t S, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int64_t MB) {
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  WorkspaceLayout w{};
  const int64_t pt = partition_tokens(S, Hkv, MB, 2);  // the most partitions any decode kernel takes
  const int64_t parts = (MB * kBlockTokens + pt - 1) / pt;
  w.tile_start_off = 0;
  w.counter_off = align(size_t(S + 1) * sizeof(int32_t));
  w.order_off = w.counter_off + 256;
  w.sched_off = w.order_off + align(size_t(kMaxSortedTiles) * kTileRecord * sizeof(int32_t));
  w.dorder_off = w.sched_off + align(size_t(2 * kMaxPrefillWorkgroups) * sizeof(int32_t));
  // the decode's work order: one record per (sequence, head group, partition)
  const int64_t units = std::min(S * (Hkv / decode_heads_per_workgroup(Hkv)) * parts, kMaxOrderedUnits);
  w.ml_off = w.dorder_off + align(size_t(kDecodeOrderHeader + units * kDecodeOrderRecord) * sizeof(int32_t));
  // split-K partials, one set per (new token, query head, partition): the
  // decode kernel's sequences use them for their partitions, and the bf16
  // prefill for the key-range pieces of its split items (the rows of the
  // prefill kernel's tokens, which the decode never touches)
  w.o_off = w.ml_off + align(size_t(T) * Hq * parts * sizeof(float2));
  w.total = w.o_off + align(size_t(T) * Hq * parts * D * sizeof(float));
  return w;
}

}  // namespace pa

namespace {

// Content checks, only with PA_VALIDATE=1 in the environment (read at each
// call). They copy the metadata to the host after the work queued on the
// stream (so a stream under graph capture cannot use them) and apply the
// rules of a flattened step: query_start_loc starts at 0, never decreases and
// ends at or before T ("Inside vLLM", section "Run forward pass": one
// super-sequence of all the step's tokens; rows past query_start_loc[S] are
// padding, as are sequences with no new token); a sequence's length is its
// cached context plus its new tokens; its first ceil(length / 16) table
// entries are pool block ids ("Serving models at scale with vLLM", section
// "PagedAttention"); each slot is negative (skipped) or inside the pool, and
// no two tokens share one.
bool validate_contents() {
  const char* e = std::getenv("PA_VALIDATE");
  return e && e[0] == '1' && e[1] == 0;
}

template <class T>
pa_status to_host(std::vector<T>& h, const T* d, size_t n, hipStream_t s) {
  h.resize(n);
  if (n == 0) return ok();
  PA_TRY(hip_status(hipMemcpyAsync(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost, s), "PA_VALIDATE copy"));
  return hip_status(hipStreamSynchronize(s), "PA_VALIDATE sync");
}

pa_status check_write_contents(const pa::WriteArgs& w, hipStream_t s) {
  std::vector<int64_t> slots;
  PA_TRY(to_host(slots, w.slots, size_t(w.T), s));
  const int64_t nslots = w.NB * pa::kBlockTokens;
  std::vector<int64_t> used;
  for (int64_t t = 0; t < w.T; ++t) {
    if (slots[t] < 0) continue;
    if (slots[t] >= nslots)
      return fail(PA_ERR_CONTENTS, "slot_mapping[%lld] = %lld is past the pool (%lld slots)", (long long)t,
                  (long long)slots[t], (long long)nslots);
    used.push_back(slots[t]);
  }
  std::sort(used.begin(), used.end());
  const auto dup = std::adjacent_find(used.begin(), used.end());
  if (dup != used.end()) return fail(PA_ERR_CONTENTS, "slot %lld is written by two tokens", (long long)*dup);
  return ok();
}

pa_status check_attention_contents(const pa::AttnArgs& a, hipStream_t s) {
  std::vector<int32_t> qsl, sl, cl, bt;
  PA_TRY(to_host(qsl, a.qsl, size_t(a.S + 1), s));
  PA_TRY(to_host(sl, a.seq_lens, size_t(a.S), s));
  PA_TRY(to_host(cl, a.ctx_lens, size_t(a.S), s));
  PA_TRY(to_host(bt, a.block_tables, a.S > 0 ? size_t((a.S - 1) * a.bt_row + a.MB) : 0, s));
  if (qsl[0] != 0) return fail(PA_ERR_CONTENTS, "query_start_loc[0] = %d, expected 0", qsl[0]);
  if (qsl[a.S] > a.T)
    return fail(PA_ERR_CONTENTS, "query_start_loc[S] = %d is past T = %lld", qsl[a.S], (long long)a.T);
  for (int64_t i = 0; i < a.S; ++i) {
    const int64_t n = int64_t(qsl[i + 1]) - qsl[i];
    if (n < 0)
      return fail(PA_ERR_CONTENTS, "query_start_loc decreases at sequence %lld (%d -> %d)", (long long)i, qsl[i],
                  qsl[i + 1]);
    if (cl[i] < 0 || int64_t(sl[i]) != cl[i] + n)
      return fail(PA_ERR_CONTENTS, "sequence %lld: seq_len %d != context_len %d + %lld new tokens", (long long)i, sl[i],
                  cl[i], (long long)n);
    const int64_t nb = (int64_t(sl[i]) + pa::kBlockTokens - 1) / pa::kBlockTokens;
    if (nb > a.MB)
      return fail(PA_ERR_CONTENTS, "sequence %lld needs %lld blocks, block_tables has %lld columns", (long long)i,
                  (long long)nb, (long long)a.MB);
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t id = bt[size_t(i * a.bt_row + j)];
      if (id < 0 || id >= a.NB)
        return fail(PA_ERR_CONTENTS, "block_tables[%lld][%lld] = %d is outside the pool (%lld blocks)", (long long)i,
                    (long long)j, id, (long long)a.NB);
    }
  }
  return ok();
}

pa_status reshape_and_cache_impl(const pa_tensor* k, const pa_tensor* v, const pa_tensor* key_cache,
                                 const pa_tensor* value_cache, const pa_tensor* slot_mapping, bool fp8, float k_scale,
                                 float v_scale, pa_stream stream) {
  pa::WriteArgs a{};
  PA_TRY(validate_write(k, v, key_cache, value_cache, slot_mapping, fp8, k_scale, v_scale, &a));
  if (a.T == 0) return ok();
  if (validate_contents()) PA_TRY(check_write_contents(a, static_cast<hipStream_t>(stream)));
  PA_TRY(hip_status(pa::launch_kv_write(a, static_cast<hipStream_t>(stream)), "kv write launch"));
  return ok();
}

pa_status attention_impl(const pa_tensor* out, const pa_tensor* q, const pa_tensor* key_cache,
                         const pa_tensor* value_cache, const pa_tensor* block_tables, const pa_tensor* query_start_loc,
                         const pa_tensor* seq_lens, const pa_tensor* context_lens, float scale, bool fp8,
                         float k_scale, float v_scale, void* workspace, size_t workspace_bytes, pa_stream stream) {
  pa::AttnArgs a{};
  PA_TRY(validate_attention(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, context_lens,
                            scale, fp8, k_scale, v_scale, workspace, workspace_bytes, &a));
  if (validate_contents()) PA_TRY(check_attention_contents(a, static_cast<hipStream_t>(stream)));
  PA_TRY(run_attention(a, static_cast<hipStream_t>(stream)));
  return ok();
}

}  // namespace

namespace pa {

pa_status step_impl(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                    const pa_tensor* key_cache, const pa_tensor* value_cache, const pa_tensor* slot_mapping,
                    const pa_tensor* block_tables, const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                    const pa_tensor* context_lens, float scale, bool fp8, float k_scale, float v_scale,
                    void* workspace, size_t workspace_bytes, pa_stream stream, bool allow_side) {
  pa::WriteArgs w{};
  pa::AttnArgs a{};
  PA_TRY(validate_write(k, v, key_cache, value_cache, slot_mapping, fp8, k_scale, v_scale, &w));
  PA_TRY(validate_attention(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, context_lens,
                            scale, fp8, k_scale, v_scale, workspace, workspace_bytes, &a));
  if (w.T != a.T)
    return fail(PA_ERR_SHAPE, "k has %lld tokens, q has %lld", (long long)w.T, (long long)a.T);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate_contents()) {
    if (w.T > 0) PA_TRY(check_write_contents(w, s));
    PA_TRY(check_attention_contents(a, s));
  }
  // Without a second stream the plan goes out in the KV write's launch.
  const bool fused = w.T > 0 && a.S > 0 && !attention_beside(a, allow_side);
  if (fused) PA_TRY(hip_status(pa::launch_write_plan(w, a, s), "kv write launch"));
  else if (w.T > 0) PA_TRY(hip_status(pa::launch_kv_write(w, s), "kv write launch"));
  PA_TRY(run_attention(a, s, allow_side, fused));
  return ok();
}

}  // namespace pa


extern "C" {

pa_status pa_reshape_and_cache(const pa_tensor* k, const pa_tensor* v, const pa_tensor* key_cache,
                               const pa_tensor* value_cache, const pa_tensor* slot_mapping, pa_stream stream) {
  return reshape_and_cache_impl(k, v, key_cache, value_cache, slot_mapping, false, 1.f, 1.f, stream);
}

pa_status pa_attention(const pa_tensor* out, const pa_tensor* q, const pa_tensor* key_cache,
                       const pa_tensor* value_cache, const pa_tensor* block_tables,
                       const pa_tensor* query_start_loc, const pa_tensor* seq_lens, const pa_tensor* context_lens,
                       float scale, void* workspace, size_t workspace_bytes, pa_stream stream) {
  return attention_impl(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, context_lens, scale,
                        false, 1.f, 1.f, workspace, workspace_bytes, stream);
}

pa_status pa_step(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                  const pa_tensor* key_cache, const pa_tensor* value_cache, const pa_tensor* slot_mapping,
                  const pa_tensor* block_tables, const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                  const pa_tensor* context_lens, float scale, void* workspace, size_t workspace_bytes,
                  pa_stream stream) {
  return pa::step_impl(out, q, k, v, key_cache, value_cache, slot_mapping, block_tables, query_start_loc, seq_lens,
                       context_lens, scale, false, 1.f, 1.f, workspace, workspace_bytes, stream, true);
}

pa_status pa_reshape_and_cache_fp8(const pa_tensor* k, const pa_tensor* v, const pa_tensor* key_cache,
                                   const pa_tensor* value_cache, const pa_tensor* slot_mapping, float k_scale,
                                   float v_scale, pa_stream stream) {
  return reshape_and_cache_impl(k, v, key_cache, value_cache, slot_mapping, true, k_scale, v_scale, stream);
}

pa_status pa_attention_fp8(const pa_tensor* out, const pa_tensor* q, const pa_tensor* key_cache,
                           const pa_tensor* value_cache, const pa_tensor* block_tables,
                           const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                           const pa_tensor* context_lens, float scale, float k_scale, float v_scale,
                           void* workspace, size_t workspace_bytes, pa_stream stream) {
  return attention_impl(out, q, key_cache, value_cache, block_tables, query_start_loc, seq_lens, context_lens, scale,
                        true, k_scale, v_scale, workspace, workspace_bytes, stream);
}

pa_status pa_step_fp8(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                      const pa_tensor* key_cache, const pa_tensor* value_cache, const pa_tensor* slot_mapping,
                      const pa_tensor* block_tables, const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                      const pa_tensor* context_lens, float scale, float k_scale, float v_scale, void* workspace,
                      size_t workspace_bytes, pa_stream stream) {
  return pa::step_impl(out, q, k, v, key_cache, value_cache, slot_mapping, block_tables, query_start_loc, seq_lens,
                       context_lens, scale, true, k_scale, v_scale, workspace, workspace_bytes, stream, true);
}

size_t pa_attention_workspace_size(int64_t num_seqs, int64_t num_tokens, int64_t num_q_heads, int64_t num_kv_heads,
                                   int64_t head_size, int64_t max_blocks_per_seq) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_size < 1 ||
      max_blocks_per_seq < 1)
    return 0;
  return pa::workspace_layout(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_size, max_blocks_per_seq).total;
}

int64_t pa_partition_tokens(int64_t num_seqs, int64_t num_kv_heads, int64_t head_size, int32_t q_dtype,
                            int32_t cache_dtype, int64_t max_blocks_per_seq) {
  const bool ok_types = (q_dtype == PA_F32 && cache_dtype == PA_F32) ||
                        (q_dtype == PA_BF16 && (cache_dtype == PA_BF16 || cache_dtype == PA_FP8_E4M3));
  if (num_seqs < 0 || num_kv_heads < 1 || max_blocks_per_seq < 1 || (head_size != 64 && head_size != 128) ||
      !ok_types)
    return 0;
  const pa::Elem elem = q_dtype == PA_F32 ? pa::Elem::F32 : pa::Elem::BF16;
  return pa::partition_tokens(num_seqs, num_kv_heads, max_blocks_per_seq,
                              pa::decode_workgroups_per_cu(elem, cache_dtype == PA_FP8_E4M3, head_size));
}

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_DTYPE: return "wrong or inconsistent element type";
    case PA_ERR_SHAPE: return "inconsistent shapes";
    case PA_ERR_STRIDE: return "unsupported layout or alignment";
    case PA_ERR_UNSUPPORTED: return "unsupported size";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "not enough free KV blocks";
    case PA_ERR_REQUEST: return "unknown request or token count";
    case PA_ERR_CONTENTS: return "device metadata invalid (PA_VALIDATE)";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_version(void) { return 100; }

}  // extern "C"
