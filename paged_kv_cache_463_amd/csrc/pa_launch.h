// Internal launcher interface between the C ABI (pa_api.cpp) and the kernel
// translation units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int32_t kKvFp8 = 3;   // DecodeParams::kv_dtype of an FP8 (e4m3) cache

struct ScatterParams {
  const void* key;
  const void* value;
  int64_t token_stride_bytes;
  void* k_cache;
  void* v_cache;
  int64_t block_stride_bytes;
  int64_t num_slots;            // num_blocks * block_size
  const int32_t* slot_mapping;
  int64_t num_tokens;
  int32_t row_bytes;            // num_kv_heads * head_dim * cache element bytes
  // FP8 (e4m3) cache only: input element type, head_dim, per-kv-head scales
  int32_t in_dtype;
  int32_t head_dim;
  const float* k_scale;
  const float* v_scale;
};

struct DecodeParams {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  int64_t block_stride_bytes;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t block_table_stride;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;                // query / output type
  int32_t kv_dtype;             // cache type: dtype, or FP8 (e4m3)
  const float* k_scale;         // FP8 cache: [num_kv_heads] dequantisation scales
  const float* v_scale;
  float scale;
  // fused decode step (single pass only): this step's token of each sequence,
  // [num_seqs][num_kv_heads][head_dim] of `dtype`, written at position L-1
  // through the table before the attention reads it; null = no write
  const void* key_new;
  const void* value_new;
  int64_t new_token_stride_bytes;
  // split-KV only
  int32_t partition_blocks;     // partition_size / 16
  int32_t max_parts;            // ceil(max_context_len / partition_size)
  int32_t max_blocks;           // blocks walked per sequence at most (set by the launcher)
  float* ws_acc;                // [num_seqs][num_q_heads][max_parts][head_dim]
  float* ws_ml;                 // [num_seqs][num_q_heads][max_parts][2]  (max, normaliser)
  int32_t* ws_ctr;              // work counter of the partition kernel (zeroed per call)
};

struct PrefillParams {
  void* out;
  const void* query;
  const int32_t* cu_q_lens;
  int32_t max_q_len;
  int64_t num_q_tokens;
  const void* k_cache;
  const void* v_cache;
  int64_t block_stride_bytes;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t block_table_stride;
  const int32_t* seq_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t causal;
  float scale;
};

struct BlockCopyParams {
  void* k_cache;
  void* v_cache;
  int64_t block_stride_bytes;
  int64_t num_blocks;
  int64_t block_bytes;          // 16 * num_kv_heads * head_dim * element bytes
  const int32_t* pairs;         // [num_pairs][2] (source, destination), device
  int64_t num_pairs;
};

hipError_t launch_reshape_and_cache(const ScatterParams& p, hipStream_t s);
hipError_t launch_reshape_and_cache_fp8(const ScatterParams& p, hipStream_t s);
constexpr int kSwapChunk = 240;              // pairs per swap launch (kernel-argument space)
struct SwapChunk {
  void* dst;                    // both pools addressable by the device
  const void* src;
  int64_t block_bytes;          // a multiple of 16
  int32_t num_pairs;            // 1 .. kSwapChunk
  int32_t pairs[kSwapChunk][2]; // (source, destination), checked on the host
};

// read-bandwidth calibration (read_probe.hip)
struct ReadProbeParams {
  const void* k_cache;
  const void* v_cache;
  int64_t block_stride_bytes;
  int64_t num_blocks;
  const int32_t* block_tables;
  int32_t block_table_stride;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t row_bytes;            // head_dim * cache element bytes (128, 256 or 512)
  int32_t partition_blocks;     // split-KV walk: partition_size / 16; 0: single-pass walk
  int32_t max_parts;            // ceil(max_context_len / partition_size) (split-KV walk)
  uint32_t* sink;
  int64_t sink_words;
};
hipError_t launch_read_probe(const ReadProbeParams& p, hipStream_t s);

hipError_t launch_copy_blocks(const BlockCopyParams& p, hipStream_t s);
hipError_t launch_swap_chunk(const SwapChunk& c, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_splitkv(const DecodeParams& p, hipStream_t s);

// Static split-KV scratch of pa_decode_splitkv_noalloc (splitkv_scratch.hip):
// its size, and its address on the current device (looked up once per device).
constexpr size_t kScratchBytes = size_t(80) << 20;
hipError_t scratch_device_ptr(void** out);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);
// chunked prefill over an FP8 (e4m3) cache: per-kv-head dequantisation scales
hipError_t launch_prefill_fp8(const PrefillParams& p, const float* k_scale, const float* v_scale, hipStream_t s);

}  // namespace pa
