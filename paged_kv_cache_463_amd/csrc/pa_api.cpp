// C ABI of the paged-attention library: argument validation and dispatch.
// Declarations, layouts and error behaviour are documented in include/pa.h.
// Validation touches no HIP API, so every error path returns before any
// device work is enqueued.
#include <algorithm>

#include "pa.h"

#include <hip/hip_runtime.h>

#include "pa_launch.h"

static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::kScratchBytes, "header and library agree on the scratch size");

namespace {

constexpr int32_t kVersion = 301;  // 0.3.1

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_DTYPE_F32: return 4;
    case PA_DTYPE_F16: return 2;
    case PA_DTYPE_BF16: return 2;
    default: return 0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool group_supported(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// The address under which the device reaches `p`, or nullptr when it cannot:
// device and managed memory as they are, pinned host memory through its mapped
// device address; pageable host memory is unknown to the runtime (the query
// fails, and its error is cleared so that it cannot surface later).
const void* device_view(const void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged || a.isManaged) return p;
  if (a.type == hipMemoryTypeHost && a.devicePointer) {
    const char* base_h = static_cast<const char*>(a.hostPointer ? a.hostPointer : p);
    return static_cast<const char*>(a.devicePointer) + (static_cast<const char*>(p) - base_h);
  }
  return nullptr;
}
void* device_view(void* p) { return const_cast<void*>(device_view(static_cast<const void*>(p))); }

// Checks shared by the attention entry points. `cache_bytes` is the cache's
// element size when it differs from the query type (1 for an FP8 cache).
int32_t check_attention_common(const void* out, const void* query, const void* k_cache,
                               const void* v_cache, int64_t block_stride, int64_t num_blocks,
                               const int32_t* block_tables, int32_t block_table_stride,
                               const int32_t* lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t dtype, int cache_bytes = 0) {
  if (elem_bytes(dtype) == 0) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 ||
      block_table_stride < 0)
    return PA_ERR_SHAPE;
  if (block_size != 16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!group_supported(num_q_heads / num_kv_heads)) return PA_ERR_UNSUPPORTED;
  if (block_stride < (int64_t)block_size * num_kv_heads * head_dim) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !lens) return PA_ERR_NULL_PTR;
  if (num_blocks == 0 || block_table_stride == 0) return PA_ERR_SHAPE;
  const int e = cache_bytes ? cache_bytes : elem_bytes(dtype);
  if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (block_stride * e) % 16 != 0)
    return PA_ERR_ALIGNMENT;
  return PA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

pa::DecodeParams make_decode_params(void* out, const void* query, const void* k_cache,
                                    const void* v_cache, int64_t block_stride, int64_t num_blocks,
                                    const int32_t* block_tables, int32_t block_table_stride,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    float scale, int32_t dtype) {
  pa::DecodeParams p{};
  p.out = out;
  p.query = query;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_stride_bytes = block_stride * elem_bytes(dtype);
  p.num_blocks = num_blocks;
  p.block_tables = block_tables;
  p.block_table_stride = block_table_stride;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.dtype = dtype;
  p.kv_dtype = dtype;
  p.scale = scale;
  return p;
}

// Turns a decode parameter block into its FP8-cache form.
void make_fp8(pa::DecodeParams& p, int64_t block_stride, const float* k_scale, const float* v_scale) {
  p.kv_dtype = pa::kKvFp8;
  p.block_stride_bytes = block_stride;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
}

// Split-KV workspace carving: fp32 partial outputs, (max, normaliser) pairs,
// the work counter; each part 256-byte aligned.
void carve_splitkv(pa::DecodeParams& p, void* workspace, int32_t mcl, int32_t partition_size) {
  p.partition_blocks = partition_size / 16;
  p.max_parts = (int32_t)ceil_div(mcl, partition_size);
  const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads * p.max_parts;
  p.ws_acc = static_cast<float*>(workspace);
  const int64_t acc_bytes = ceil_div(rows * p.head_dim * 4, 256) * 256;
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + acc_bytes);
  p.ws_ctr = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + acc_bytes +
                                        ceil_div(rows * 2 * 4, 256) * 256);
}

}  // namespace

extern "C" {

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL_PTR: return "PA_ERR_NULL_PTR: a required pointer is NULL";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown or unsupported dtype";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent size or stride";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: block_size, head_dim or group not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: split-KV workspace missing or too small";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the call needs more split-KV scratch than the library's static array holds";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP launch error";
    case PA_ERR_ALIGNMENT: return "PA_ERR_ALIGNMENT: pointer or stride not 16-byte aligned";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free blocks";
    case PA_ERR_SEQUENCE: return "PA_ERR_SEQUENCE: unknown request id, or one already in use";
    default: return "unknown pa_status_t";
  }
}

int32_t pa_version(void) { return kVersion; }

int32_t pa_reshape_and_cache(const void* key, const void* value, int64_t kv_token_stride,
                             void* k_cache, void* v_cache, int64_t block_stride,
                             int64_t num_blocks, const int32_t* slot_mapping, int64_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t dtype, void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0) return PA_ERR_SHAPE;
  if (block_size != 16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (kv_token_stride < row || block_stride < block_size * row) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL_PTR;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (kv_token_stride * e) % 16 != 0 || (block_stride * e) % 16 != 0)
    return PA_ERR_ALIGNMENT;
  pa::ScatterParams p{};
  p.key = key;
  p.value = value;
  p.token_stride_bytes = kv_token_stride * e;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_stride_bytes = block_stride * e;
  p.num_slots = num_blocks * block_size;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.row_bytes = (int32_t)(row * e);
  return hip_status(pa::launch_reshape_and_cache(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_copy_blocks(void* k_cache, void* v_cache, int64_t block_stride, int64_t num_blocks,
                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype, const int32_t* pairs,
                       int64_t num_pairs, void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0) return PA_ERR_DTYPE;
  if (num_pairs < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0) return PA_ERR_SHAPE;
  const int64_t block_elems = (int64_t)16 * num_kv_heads * head_dim;
  if (block_stride < block_elems || num_pairs > 0x7FFFFFFF) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_NULL_PTR;
  if (!aligned16(k_cache) || !aligned16(v_cache) || (block_stride * e) % 16 != 0 || (block_elems * e) % 16 != 0)
    return PA_ERR_ALIGNMENT;
  pa::BlockCopyParams p{};
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_stride_bytes = block_stride * e;
  p.num_blocks = num_blocks;
  p.block_bytes = block_elems * e;
  p.pairs = pairs;
  p.num_pairs = num_pairs;
  return hip_status(pa::launch_copy_blocks(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_swap_blocks(void* dst_pool, int64_t dst_blocks, const void* src_pool, int64_t src_blocks,
                       int64_t block_bytes, const int64_t* pairs, int64_t num_pairs, void* stream) {
  if (num_pairs < 0 || dst_blocks < 0 || src_blocks < 0 || block_bytes <= 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dst_pool || !src_pool || !pairs) return PA_ERR_NULL_PTR;
  for (int64_t i = 0; i < num_pairs; ++i) {         // check everything before moving anything
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return PA_ERR_SHAPE;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // both pools addressable by the device (device memory, or pinned host memory
  // mapped into its address space): the swap kernel moves every pair in a few
  // launches; otherwise the copy engine moves runs of consecutive pairs
  void* dview = device_view(dst_pool);
  const void* sview = device_view(src_pool);
  if (dview && sview && block_bytes % 16 == 0 && aligned16(dview) && aligned16(sview) &&
      dst_blocks <= 0x7FFFFFFF && src_blocks <= 0x7FFFFFFF) {
    pa::SwapChunk c{};
    c.dst = dview;
    c.src = sview;
    c.block_bytes = block_bytes;
    for (int64_t i0 = 0; i0 < num_pairs; i0 += pa::kSwapChunk) {
      c.num_pairs = (int32_t)std::min<int64_t>(pa::kSwapChunk, num_pairs - i0);
      for (int32_t k = 0; k < c.num_pairs; ++k) {
        c.pairs[k][0] = (int32_t)pairs[2 * (i0 + k)];
        c.pairs[k][1] = (int32_t)pairs[2 * (i0 + k) + 1];
      }
      if (pa::launch_swap_chunk(c, st) != hipSuccess) return PA_ERR_HIP;
    }
    return PA_OK;
  }
  int64_t i = 0;
  while (i < num_pairs) {                           // merge runs of consecutive pairs
    const int64_t s0 = pairs[2 * i], d0 = pairs[2 * i + 1];
    int64_t n = 1;
    while (i + n < num_pairs && pairs[2 * (i + n)] == s0 + n && pairs[2 * (i + n) + 1] == d0 + n) ++n;
    const hipError_t e = hipMemcpyAsync(static_cast<char*>(dst_pool) + d0 * block_bytes,
                                        static_cast<const char*>(src_pool) + s0 * block_bytes,
                                        (size_t)(n * block_bytes), hipMemcpyDefault, st);
    if (e != hipSuccess) return PA_ERR_HIP;
    i += n;
  }
  return PA_OK;
}

int32_t pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                  int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                  int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, float scale, int32_t dtype, void* stream) {
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, context_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  pa::DecodeParams p = make_decode_params(out, query, k_cache, v_cache, block_stride, num_blocks,
                                          block_tables, block_table_stride, context_lens,
                                          num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                                          dtype);
  return hip_status(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_splitkv_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0 ||
      partition_size <= 0)
    return 0;
  const int64_t parts = ceil_div(max_context_len, partition_size);
  const int64_t rows = (int64_t)num_seqs * num_q_heads * parts;
  // fp32 partial outputs, then (max, normaliser) pairs, then the work counter;
  // each part 256-byte aligned
  const int64_t acc_bytes = ceil_div(rows * head_dim * 4, 256) * 256;
  const int64_t ml_bytes = ceil_div(rows * 2 * 4, 256) * 256;
  return (size_t)(acc_bytes + ml_bytes + 256);
}

int32_t pa_decode_splitkv(void* out, const void* query, const void* k_cache, const void* v_cache,
                          int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                          int32_t block_table_stride, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                          int32_t max_context_len, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, context_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % 16 != 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  // all-empty batches still get their zero rows written by the merge kernel
  const int32_t mcl = max_context_len > 0 ? max_context_len : 1;
  const size_t need = pa_decode_splitkv_workspace_bytes(num_seqs, num_q_heads, head_dim, mcl,
                                                        partition_size);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_ALIGNMENT;
  pa::DecodeParams p = make_decode_params(out, query, k_cache, v_cache, block_stride, num_blocks,
                                          block_tables, block_table_stride, context_lens,
                                          num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                                          dtype);
  carve_splitkv(p, workspace, mcl, partition_size);
  return hip_status(pa::launch_decode_splitkv(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_splitkv_noalloc(void* out, const void* query, const void* k_cache, const void* v_cache,
                                  int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                                  int32_t block_table_stride, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                                  int32_t max_context_len, int32_t partition_size, void* stream) {
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, context_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % 16 != 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  const int32_t mcl = max_context_len > 0 ? max_context_len : 1;
  if (pa_decode_splitkv_workspace_bytes(num_seqs, num_q_heads, head_dim, mcl, partition_size) >
      pa::kScratchBytes)
    return PA_ERR_SCRATCH;
  void* scratch = nullptr;                  // this device's copy of the static array
  if (pa::scratch_device_ptr(&scratch) != hipSuccess) return PA_ERR_HIP;
  pa::DecodeParams p = make_decode_params(out, query, k_cache, v_cache, block_stride, num_blocks,
                                          block_tables, block_table_stride, context_lens,
                                          num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                                          dtype);
  carve_splitkv(p, scratch, mcl, partition_size);
  return hip_status(pa::launch_decode_splitkv(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_read_kv_rows(const void* k_cache, const void* v_cache, int64_t block_stride, int64_t num_blocks,
                        const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t cache_elem_bytes,
                        int32_t max_context_len, int32_t partition_size, uint32_t* sink, int64_t sink_words,
                        void* stream) {
  if (num_seqs < 0 || num_kv_heads <= 0 || num_blocks < 0 || block_table_stride < 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (cache_elem_bytes != 1 && cache_elem_bytes != 2 && cache_elem_bytes != 4) return PA_ERR_DTYPE;
  if (partition_size < 0 || partition_size % 16 != 0) return PA_ERR_SHAPE;
  if (block_stride < (int64_t)16 * num_kv_heads * head_dim) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !sink) return PA_ERR_NULL_PTR;
  if (num_blocks == 0 || block_table_stride == 0 || sink_words <= 0) return PA_ERR_SHAPE;
  if (partition_size > 0 && num_seqs > 1024) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k_cache) || !aligned16(v_cache) || (block_stride * cache_elem_bytes) % 16 != 0)
    return PA_ERR_ALIGNMENT;
  pa::ReadProbeParams p{};
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_stride_bytes = block_stride * cache_elem_bytes;
  p.num_blocks = num_blocks;
  p.block_tables = block_tables;
  p.block_table_stride = block_table_stride;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_kv_heads = num_kv_heads;
  p.row_bytes = head_dim * cache_elem_bytes;
  p.partition_blocks = partition_size / 16;
  p.max_parts = partition_size > 0 ? (int32_t)ceil_div(max_context_len > 0 ? max_context_len : 1, partition_size) : 0;
  p.sink = sink;
  p.sink_words = sink_words;
  return hip_status(pa::launch_read_probe(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_step(void* out, const void* query, const void* key_new, const void* value_new,
                       int64_t kv_token_stride, void* k_cache, void* v_cache, int64_t block_stride,
                       int64_t num_blocks, const int32_t* block_tables, int32_t block_table_stride,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                       int32_t dtype, void* stream) {
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, context_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  const int e = elem_bytes(dtype);
  if (!key_new || !value_new) return PA_ERR_NULL_PTR;
  if (kv_token_stride < (int64_t)num_kv_heads * head_dim) return PA_ERR_SHAPE;
  if (!aligned16(key_new) || !aligned16(value_new) || (kv_token_stride * e) % 16 != 0)
    return PA_ERR_ALIGNMENT;
  pa::DecodeParams p = make_decode_params(out, query, k_cache, v_cache, block_stride, num_blocks,
                                          block_tables, block_table_stride, context_lens,
                                          num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                                          dtype);
  p.key_new = key_new;
  p.value_new = value_new;
  p.new_token_stride_bytes = kv_token_stride * e;
  return hip_status(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_step_fp8(void* out, const void* query, const void* key_new, const void* value_new,
                           int64_t kv_token_stride, void* k_cache, void* v_cache,
                           int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                           int32_t block_table_stride, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, float scale,
                           const float* k_scale, const float* v_scale, int32_t dtype,
                           void* stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, context_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype, 1);
  if (st != PA_OK || num_seqs == 0) return st;
  const int e = elem_bytes(dtype);
  if (!key_new || !value_new || !k_scale || !v_scale) return PA_ERR_NULL_PTR;
  if (kv_token_stride < (int64_t)num_kv_heads * head_dim) return PA_ERR_SHAPE;
  if (!aligned16(key_new) || !aligned16(value_new) || (kv_token_stride * e) % 16 != 0)
    return PA_ERR_ALIGNMENT;
  pa::DecodeParams p = make_decode_params(out, query, k_cache, v_cache, block_stride, num_blocks,
                                          block_tables, block_table_stride, context_lens,
                                          num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                                          dtype);
  make_fp8(p, block_stride, k_scale, v_scale);
  p.key_new = key_new;
  p.value_new = value_new;
  p.new_token_stride_bytes = kv_token_stride * e;
  return hip_status(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_reshape_and_cache_fp8(const void* key, const void* value, int64_t kv_token_stride,
                                 void* k_cache, void* v_cache, int64_t block_stride,
                                 int64_t num_blocks, const int32_t* slot_mapping, int64_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 const float* k_scale, const float* v_scale, int32_t dtype,
                                 void* stream) {
  const int e = elem_bytes(dtype);
  if (e == 0) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0) return PA_ERR_SHAPE;
  if (block_size != 16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (kv_token_stride < row || block_stride < block_size * row) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale)
    return PA_ERR_NULL_PTR;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (kv_token_stride * e) % 16 != 0 || block_stride % 16 != 0)
    return PA_ERR_ALIGNMENT;
  pa::ScatterParams p{};
  p.key = key;
  p.value = value;
  p.token_stride_bytes = kv_token_stride * e;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_stride_bytes = block_stride;
  p.num_slots = num_blocks * block_size;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.row_bytes = (int32_t)row;
  p.in_dtype = dtype;
  p.head_dim = head_dim;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  return hip_status(pa::launch_reshape_and_cache_fp8(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_fp8(void* out, const void* query, const void* k_cache, const void* v_cache,
                      int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                      int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, float scale, const float* k_scale, const float* v_scale,
                      int32_t dtype, void* stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, context_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype, 1);
  if (st != PA_OK || num_seqs == 0) return st;
  if (!k_scale || !v_scale) return PA_ERR_NULL_PTR;
  pa::DecodeParams p = make_decode_params(out, query, k_cache, v_cache, block_stride, num_blocks,
                                          block_tables, block_table_stride, context_lens,
                                          num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                                          dtype);
  make_fp8(p, block_stride, k_scale, v_scale);
  return hip_status(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_splitkv_fp8(void* out, const void* query, const void* k_cache,
                              const void* v_cache, int64_t block_stride, int64_t num_blocks,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              float scale, const float* k_scale, const float* v_scale,
                              int32_t dtype, int32_t max_context_len, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PA_DTYPE_F16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, context_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype, 1);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % 16 != 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!k_scale || !v_scale) return PA_ERR_NULL_PTR;
  const int32_t mcl = max_context_len > 0 ? max_context_len : 1;
  const size_t need = pa_decode_splitkv_workspace_bytes(num_seqs, num_q_heads, head_dim, mcl,
                                                        partition_size);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_ALIGNMENT;
  pa::DecodeParams p = make_decode_params(out, query, k_cache, v_cache, block_stride, num_blocks,
                                          block_tables, block_table_stride, context_lens,
                                          num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                                          dtype);
  make_fp8(p, block_stride, k_scale, v_scale);
  carve_splitkv(p, workspace, mcl, partition_size);
  return hip_status(pa::launch_decode_splitkv(p, static_cast<hipStream_t>(stream)));
}

// Shared argument checks and parameter block of the two prefill entry points;
// cache_bytes = 0: the cache has the query's type, 1: FP8 codes.
static int32_t prefill_params(pa::PrefillParams& p, void* out, const void* query, const int32_t* cu_q_lens,
                              int32_t max_q_len, int64_t num_q_tokens, const void* k_cache,
                              const void* v_cache, int64_t block_stride, int64_t num_blocks,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                              int32_t causal, int32_t dtype, int cache_bytes, bool& empty) {
  empty = false;
  int32_t st = check_attention_common(out, query, k_cache, v_cache, block_stride, num_blocks,
                                      block_tables, block_table_stride, seq_lens, num_seqs,
                                      num_q_heads, num_kv_heads, head_dim, block_size, dtype, cache_bytes);
  if (st != PA_OK) return st;
  if (dtype != PA_DTYPE_BF16 && dtype != PA_DTYPE_F16) return PA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return PA_ERR_SHAPE;
  if (max_q_len < 0 || num_q_tokens < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_q_tokens == 0 || max_q_len == 0) {
    empty = true;
    return PA_OK;
  }
  if (!cu_q_lens) return PA_ERR_NULL_PTR;
  p = pa::PrefillParams{};
  p.out = out;
  p.query = query;
  p.cu_q_lens = cu_q_lens;
  p.max_q_len = max_q_len;
  p.num_q_tokens = num_q_tokens;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_stride_bytes = block_stride * (cache_bytes ? cache_bytes : elem_bytes(dtype));
  p.num_blocks = num_blocks;
  p.block_tables = block_tables;
  p.block_table_stride = block_table_stride;
  p.seq_lens = seq_lens;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.dtype = dtype;
  p.causal = causal;
  p.scale = scale;
  return PA_OK;
}

int32_t pa_prefill_chunked(void* out, const void* query, const int32_t* cu_q_lens,
                           int32_t max_q_len, int64_t num_q_tokens, const void* k_cache,
                           const void* v_cache, int64_t block_stride, int64_t num_blocks,
                           const int32_t* block_tables, int32_t block_table_stride,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           float scale, int32_t causal, int32_t dtype, void* stream) {
  pa::PrefillParams p;
  bool empty;
  const int32_t st = prefill_params(p, out, query, cu_q_lens, max_q_len, num_q_tokens, k_cache, v_cache,
                                    block_stride, num_blocks, block_tables, block_table_stride, seq_lens,
                                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, scale, causal,
                                    dtype, 0, empty);
  if (st != PA_OK || empty) return st;
  hipError_t e = pa::launch_prefill(p, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return PA_ERR_UNSUPPORTED;
  return hip_status(e);
}

int32_t pa_prefill_chunked_fp8(void* out, const void* query, const int32_t* cu_q_lens,
                               int32_t max_q_len, int64_t num_q_tokens, const void* k_cache,
                               const void* v_cache, int64_t block_stride, int64_t num_blocks,
                               const int32_t* block_tables, int32_t block_table_stride,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               float scale, int32_t causal, const float* k_scale, const float* v_scale,
                               int32_t dtype, void* stream) {
  pa::PrefillParams p;
  bool empty;
  const int32_t st = prefill_params(p, out, query, cu_q_lens, max_q_len, num_q_tokens, k_cache, v_cache,
                                    block_stride, num_blocks, block_tables, block_table_stride, seq_lens,
                                    num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, scale, causal,
                                    dtype, 1, empty);
  if (st != PA_OK || empty) return st;
  if (!k_scale || !v_scale) return PA_ERR_NULL_PTR;
  hipError_t e = pa::launch_prefill_fp8(p, k_scale, v_scale, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return PA_ERR_UNSUPPORTED;
  return hip_status(e);
}

}  // extern "C"
