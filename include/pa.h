/*
 * pa.h -- C ABI of libpa.so: paged attention over a block-paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (as stated across the pages this library implements):
 *  - The KV cache is one pool of fixed-size blocks of 16 token slots; a block
 *    of a standard transformer layer holds 2 (K and V) x 16 x num_kv_heads x
 *    head_size elements ("Inside vLLM: Anatomy of a High-Throughput LLM
 *    Inference System", section "LLM Engine & Engine Core", KV cache
 *    manager; "Serving models at scale with vLLM", section "PagedAttention").
 *  - Each sequence reaches its blocks through a block table that lists its
 *    physical blocks in order: key position j sits in block
 *    block_tables[s][j / 16], slot j % 16 ("Serving models at scale with
 *    vLLM", section "PagedAttention").
 *  - New tokens' K/V are scattered into the pool through a flat slot_mapping
 *    built while preparing the step's inputs ("Inside vLLM", section "Run
 *    forward pass", step 2).
 *  - One step runs over all sequences flattened into one super-sequence;
 *    each sequence attends only to its own tokens ("Inside vLLM", "Run
 *    forward pass", step 3). Sequences with one new token are decodes; longer
 *    ones are (chunks of) prefills whose tokens also see everything already
 *    cached for that sequence ("Serving models at scale with vLLM", section
 *    "Chunked prefill"). Decodes and prefill chunks mix in one step
 *    ("Inside vLLM", section "Scheduler").
 *
 * Conventions for every call:
 *  - Memory: every tensor is device memory owned by the caller; the library
 *    never allocates, frees or keeps pointers to caller memory. Scratch space
 *    comes from the caller through `workspace`.
 *  - Ordering: calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *    default stream). pa_step orders the KV write before attention on that
 *    stream. No call synchronises the device or copies device data to the host.
 *    For large bf16 batches that mix decodes and prefill chunks, pa_attention
 *    and pa_step run the chunked prefill on a stream of the library's own
 *    (one per host thread and device, created on first use, kept for the
 *    life of the process, default priority), forked from `stream` and joined
 *    back into it with events: the call's work still starts after, and ends
 *    before, whatever is queued around it on `stream`, and it can be captured
 *    in a HIP graph from `stream`.
 *  - Errors: host-side checks of the descriptors (null pointers, element
 *    types, ranks, extents, strides, alignment, supported sizes, workspace
 *    size) return a pa_status before anything is launched; the text of the
 *    last failure of the calling thread is in pa_last_error(). Launch
 *    failures return PA_ERR_HIP. Device-side contents (ids, lengths, slots)
 *    are not validated by default: values outside their documented range give
 *    unspecified results, but every device access stays inside the tensors
 *    passed in (ids and lengths are clamped, out-of-range slots skipped).
 *    With PA_VALIDATE=1 in the environment (read at each call), each call
 *    first copies its metadata to the host, after the work already queued on
 *    `stream` (so not under graph capture), and returns PA_ERR_CONTENTS,
 *    launching nothing, unless: query_start_loc[0] = 0, query_start_loc
 *    never decreases and query_start_loc[S] <= T (a sequence may have no new
 *    token; rows past query_start_loc[S] are padding); seq_lens =
 *    context_lens + new tokens with context_lens >= 0; ceil(seq_len / 16) <=
 *    max blocks and those table entries lie in [0, num_blocks); every slot
 *    is negative or below num_blocks * 16, and no two tokens share a slot.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_DTYPE = 2,       /* element types wrong or inconsistent */
  PA_ERR_SHAPE = 3,       /* ranks or extents inconsistent */
  PA_ERR_STRIDE = 4,      /* layout not supported (inner dim not contiguous, misaligned) */
  PA_ERR_UNSUPPORTED = 5, /* block size != 16, head_size not 64/128, head ratio > 16 */
  PA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than pa_attention_workspace_size() */
  PA_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
  PA_ERR_NO_BLOCKS = 8,   /* KV manager: too few free blocks; nothing changed */
  PA_ERR_REQUEST = 9,     /* KV manager: unknown or duplicate request id, or a token count it does not hold */
  PA_ERR_CONTENTS = 10    /* PA_VALIDATE=1 only: block ids, lengths, query_start_loc or slots invalid */
} pa_status;

/* PA_FP8_E4M3: OCP FP8 E4M3 codes (1 byte: sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; no infinities; 0x7F / 0xFF are NaN; largest finite
 * magnitude 448). Only for key_cache / value_cache, through the _fp8 calls. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_I32 = 2, PA_I64 = 3, PA_FP8_E4M3 = 4 } pa_dtype;

#define PA_MAX_DIMS 4

/* A strided view of device memory. Strides are in elements. */
typedef struct {
  void* data;
  int32_t dtype; /* pa_dtype */
  int32_t ndim;
  int64_t shape[PA_MAX_DIMS];
  int64_t stride[PA_MAX_DIMS];
} pa_tensor;

/* hipStream_t, passed as an opaque pointer so this header needs no HIP headers. */
typedef void* pa_stream;

/*
 * KV write. For every token t with slot = slot_mapping[t] in [0, NB * 16):
 *   key_cache[slot / 16][slot % 16][:][:]   = k[t][:][:]
 *   value_cache[slot / 16][slot % 16][:][:] = v[t][:][:]
 * as a bitwise copy. Negative slots are skipped (padding tokens). Slots past
 * the pool are skipped too. Two tokens with the same slot race.
 *
 *   k, v           [T, Hkv, D]  f32 or bf16; last dim contiguous
 *   key_cache,     [NB, 16, Hkv, D] same dtype; the two halves of one pool
 *   value_cache    [NB, 2, 16, Hkv, D] (pool[:, 0] and pool[:, 1]) or any
 *                  layout with contiguous last dim and 16-byte aligned rows
 *   slot_mapping   [T] int64
 * Cite: "Inside vLLM", section "Run forward pass", step 2 (slot_mapping);
 * section "Prefix Caching" (the forward pass fills the paged KV cache).
 */
pa_status pa_reshape_and_cache(const pa_tensor* k, const pa_tensor* v, const pa_tensor* key_cache,
                               const pa_tensor* value_cache, const pa_tensor* slot_mapping, pa_stream stream);

/*
 * Attention over the flattened super-sequence. Sequence s owns query rows
 * t in [query_start_loc[s], query_start_loc[s + 1]); its i-th row sits at
 * position context_lens[s] + i and attends keys j <= context_lens[s] + i
 * (and j < seq_lens[s] = context_lens[s] + query length), read through
 * block_tables[s]. Query head h reads KV head h / (Hq / Hkv).
 *   out[t][h] = sum_j softmax_j(scale * q[t][h] . K[j]) V[j]
 * Softmax and accumulation are fp32; out is rounded to its dtype.
 *
 *   out            [T, Hq, D]   same dtype as q; written, rows of sequences
 *                               with no query rows untouched
 *   q              [T, Hq, D]   f32 or bf16; last dim contiguous
 *   key_cache,     [NB, 16, Hkv, D] as for pa_reshape_and_cache
 *   value_cache
 *   block_tables   [S, MB] int32; entries past ceil(seq_lens[s] / 16) unread
 *   query_start_loc[S + 1] int32; query_start_loc[0] = 0, non-decreasing,
 *                               query_start_loc[S] <= T
 *   seq_lens       [S] int32   keys of each sequence incl. its new tokens
 *   context_lens   [S] int32   keys cached before this step's tokens
 *   workspace      device scratch of at least pa_attention_workspace_size()
 *                  bytes, 256-byte aligned; contents need no initialisation
 *                  and are overwritten. Concurrent calls need separate ones.
 * Supported: D in {64, 128}; Hq % Hkv == 0 and Hq / Hkv <= 16.
 * Cite: "Inside vLLM", section "Run forward pass", step 3 (one flattened
 * super-sequence, each sequence masked to its own tokens; the model runner
 * prepares the block tables and context lengths); "Serving models at scale
 * with vLLM", section "PagedAttention" (a block table lists a request's
 * blocks in order) and section "Chunked prefill" (a chunk's tokens attend
 * the earlier chunks' K/V read back from the cache, and each token only the
 * tokens before it).
 */
pa_status pa_attention(const pa_tensor* out, const pa_tensor* q, const pa_tensor* key_cache,
                       const pa_tensor* value_cache, const pa_tensor* block_tables,
                       const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                       const pa_tensor* context_lens, float scale, void* workspace, size_t workspace_bytes,
                       pa_stream stream);

/*
 * One step: pa_reshape_and_cache(k, v, ...) then pa_attention(...), in that
 * order on `stream`. Arguments as above; k, v, q and slot_mapping share T.
 * Cite: "Inside vLLM", section "Run forward pass" (prepare inputs, then the
 * forward pass over the super-sequence); ngrok, section "Chunked prefill"
 * (a chunk's tokens read the K/V already in the cache).
 */
pa_status pa_step(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                  const pa_tensor* key_cache, const pa_tensor* value_cache, const pa_tensor* slot_mapping,
                  const pa_tensor* block_tables, const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                  const pa_tensor* context_lens, float scale, void* workspace, size_t workspace_bytes,
                  pa_stream stream);

/*
 * 8-bit KV pool. The pages name 8-bit quantization of the KV cache, which
 * halves the bytes every decode step reads, without fixing a format
 * ("Serving models at scale with vLLM", section on quantization): here the
 * pool holds PA_FP8_E4M3 codes with one fp32 scale for all keys and one for
 * all values.
 *  - pa_reshape_and_cache_fp8 stores code = nearest(x / k_scale) for each
 *    element x of k (v / v_scale for v): the quotient is an IEEE fp32
 *    division; nearest rounds to the closest code, ties to the even code,
 *    magnitudes above 448 to +-448 (the sign kept), NaN to 0x7F. Negative
 *    or past-the-pool slots are skipped as in pa_reshape_and_cache.
 *  - pa_attention_fp8 / pa_step_fp8 read a key element back as
 *    value(code) * k_scale and a value element as value(code) * v_scale
 *    (exact), and otherwise compute what pa_attention / pa_step compute.
 *   k, v, q, out   bf16 (q, out) and bf16 or f32 (k, v)
 *   key_cache,     [NB, 16, Hkv, D] PA_FP8_E4M3, rows 16-byte aligned
 *   value_cache
 *   k_scale,       finite and > 0
 *   v_scale
 * Other arguments, errors and ordering as for the calls above; the f32/bf16
 * calls reject an fp8 cache with PA_ERR_DTYPE.
 */
pa_status pa_reshape_and_cache_fp8(const pa_tensor* k, const pa_tensor* v, const pa_tensor* key_cache,
                                   const pa_tensor* value_cache, const pa_tensor* slot_mapping, float k_scale,
                                   float v_scale, pa_stream stream);
pa_status pa_attention_fp8(const pa_tensor* out, const pa_tensor* q, const pa_tensor* key_cache,
                           const pa_tensor* value_cache, const pa_tensor* block_tables,
                           const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                           const pa_tensor* context_lens, float scale, float k_scale, float v_scale,
                           void* workspace, size_t workspace_bytes, pa_stream stream);
pa_status pa_step_fp8(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                      const pa_tensor* key_cache, const pa_tensor* value_cache, const pa_tensor* slot_mapping,
                      const pa_tensor* block_tables, const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                      const pa_tensor* context_lens, float scale, float k_scale, float v_scale, void* workspace,
                      size_t workspace_bytes, pa_stream stream);

/*
 * pa_step without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. It computes what pa_step computes, with the same
 * arguments minus the workspace, and calls no allocating routine of any
 * library. Its scratch space is a fixed array of PA_NOALLOC_SCRATCH_BYTES in
 * the library's device memory, one per GPU, held until the process ends.
 *  - A step whose pa_attention_workspace_size() exceeds
 *    PA_NOALLOC_SCRATCH_BYTES is rejected with PA_ERR_WORKSPACE before
 *    anything is launched (use pa_step with a workspace then).
 *  - Every launch stays on `stream`: no stream or event of the library's own
 *    is created or used (large mixed batches run their prefill after the
 *    decode instead of beside it).
 *  - All calls on one GPU share its array, so calls that overlap in time on
 *    one GPU (two streams, two host threads) race; serialise them.
 *  - The array needs no initialisation: every call rewrites what it reads.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_step_noalloc(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k, const pa_tensor* v,
                          const pa_tensor* key_cache, const pa_tensor* value_cache, const pa_tensor* slot_mapping,
                          const pa_tensor* block_tables, const pa_tensor* query_start_loc, const pa_tensor* seq_lens,
                          const pa_tensor* context_lens, float scale, pa_stream stream);

/*
 * Bytes of workspace pa_attention / pa_step need for these extents (the
 * split-K partial results, one set per new token of the sequences the decode
 * kernel attends -- those whose query length times Hq / Hkv is at most 16 --
 * the prefill tile list, and the decode's work order).
 * Returns 0 for invalid extents.
 */
size_t pa_attention_workspace_size(int64_t num_seqs, int64_t num_tokens, int64_t num_q_heads,
                                   int64_t num_kv_heads, int64_t head_size, int64_t max_blocks_per_seq);

/*
 * Tokens per split-K decode partition that pa_attention / pa_step choose for
 * these extents and element types (a multiple of 16): the largest that still
 * gives one round of decode workgroups on the longest sequences the block
 * table allows, as many as the device's CUs hold at once. q_dtype is PA_F32
 * or PA_BF16; cache_dtype is q_dtype, or PA_FP8_E4M3 with PA_BF16 queries.
 * Without a device (the occupancy query fails) it assumes two workgroups per
 * CU. Returns 0 for invalid arguments.
 */
int64_t pa_partition_tokens(int64_t num_seqs, int64_t num_kv_heads, int64_t head_size, int32_t q_dtype,
                            int32_t cache_dtype, int64_t max_blocks_per_seq);

/* Static description of a status code. */
const char* pa_status_string(pa_status status);

/* Text of the last error on the calling thread ("" if none). */
const char* pa_last_error(void);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
