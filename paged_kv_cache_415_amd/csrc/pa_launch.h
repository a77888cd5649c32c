// Internal interface between the host-side C ABI (pa_api.cpp) and the
// kernel translation units.  Parameters travel to the kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Element-type codes; numerically equal to the public pa_dtype values.
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3, kI8 = 4 };

constexpr int kProbeBlocks = 2048;

struct ScatterParams {
  const void* key;
  const void* value;
  void* k_pool;
  void* v_pool;
  const int64_t* slot_mapping;
  int64_t key_stride;    // elements between consecutive tokens of `key`
  int64_t value_stride;
  int num_tokens;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int src_dtype;
  int cache_dtype;     // K pool element type
  int v_cache_dtype;   // V pool element type
  int src_elem_bytes;
  float k_scale;
  float v_scale;
  const float* k_scales;   // int8 cache: [num_blocks][num_kv_heads] per-block scales
  const float* v_scales;
};

struct CopyParams {
  void* k_pool;
  void* v_pool;
  const int64_t* pairs;
  int64_t block_bytes;
  int num_pairs;
};

// Copy of the first rows of blocks: for each triple (src, dst, n), rows
// [0, n) of every KV head of block dst become those of block src.
struct CopyRowsParams {
  void* k_pool;
  void* v_pool;
  const int64_t* triples;
  int64_t row_bytes;
  int num_kv_heads;
  int block_size;
  int num_pairs;
};

// Whole-block copies applied to the K and V pools of several layers; the
// pool pointers are device arrays of num_layers entries.
struct CopyLayersParams {
  void* const* k_pools;
  void* const* v_pools;
  const int64_t* pairs;
  int64_t block_bytes;
  int num_pairs;
  int num_layers;
};

// Block moves from one pool to another (either may be host memory mapped
// for device access): block pairs[2p + 1] of dst = block pairs[2p] of src.
struct SwapParams {
  void* dst;
  const void* src;
  const int64_t* pairs;
  int64_t block_bytes;
  int num_pairs;
};

// How a decode call cuts each (sequence, KV head) pair's context into the
// segments that single waves process.  Units are 32-token steps.
enum : int {
  kSplitBalanced = 0,  // the batch's units are cut into equal contiguous ranges, one per wave
  kSplitFixed = 1,     // fixed partitions of `chunk` units from each sequence's start
  kSplitNone = 2       // every pair is processed whole by one wave
};

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int* block_tables;
  const int* seq_lens;
  float* part_o;       // [S][Hq][max_parts][D]  unnormalised partial outputs
  float* part_m;       // [S][Hq][max_parts]     running max (log2 domain)
  float* part_l;       // [S][Hq][max_parts]     sum of exponentials
  int* nparts;         // [S][Hkv]               segments of each pair
  float qk_scale_log2; // scale * k_scale * log2(e)
  float v_scale;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int head_dim;
  int block_size;
  int max_blocks;      // block-table row length
  int max_len;         // clamp for seq_lens: min(max_seq_len, max_blocks * block_size)
  int mode;            // kSplit*
  int chunk;           // units: fixed partition length, or the shortest balanced range
  int max_parts;       // partial slots per (sequence, query head)
  int local_slots;     // LDS slots per workgroup for partials merged on the CU (0: none)
  int kstage_off;      // byte offset in LDS of the waves' 8-bit K staging (4 KB per wave)
  int q_dtype;
  int cache_dtype;     // K pool element type
  int v_cache_dtype;   // V pool element type (the same, or QT beside an fp8 K pool)
  const float* k_scales;   // int8 cache: [num_blocks][num_kv_heads] per-block scales
  const float* v_scales;
  // append: each sequence's newest token [S][Hkv][D] (row s at s * stride elements)
  const void* new_k;
  const void* new_v;
  int64_t new_k_stride;
  int64_t new_v_stride;
};

struct PrefillParams {
  void* out;
  const void* q;
  const int* query_start_loc;
  const void* k_pool;
  const void* v_pool;
  const int* block_tables;
  const int* seq_lens;
  float qk_scale_log2;
  float v_scale;
  int num_seqs;
  int total_q;
  int max_q_len;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int head_dim;
  int block_size;
  int max_blocks;
  int q_dtype;
  int cache_dtype;     // K and V pools: q_dtype, or fp8 / int8 beside 16-bit queries
  const float* k_scales;   // int8 cache: [num_blocks][num_kv_heads] per-block scales
  const float* v_scales;
};

// Index checks (flags numerically equal to the public pa_check_flag values).
enum : int { kCheckBlockId = 1, kCheckLength = 2, kCheckSlot = 4, kCheckChunk = 8 };

struct CheckParams {
  const int* block_tables;      // tables check (slots == nullptr)
  const int* seq_lens;
  const int* query_start_loc;   // optional
  const int64_t* slots;         // slots check
  int* err;                     // device int32[3]
  int num_items;                // sequences or tokens
  int max_blocks;
  int block_size;
  int num_blocks;
  int max_len;
  int total;                    // total query tokens (chunk check)
};

hipError_t launch_scatter(const ScatterParams& p, hipStream_t stream);
hipError_t launch_check(const CheckParams& p, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream);
hipError_t launch_copy_rows(const CopyRowsParams& p, hipStream_t stream);
hipError_t launch_copy_layers(const CopyLayersParams& p, hipStream_t stream);
hipError_t launch_swap_blocks(const SwapParams& p, hipStream_t stream);
hipError_t launch_decode_attention(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
// One launch over a mixed step's prefill query tiles and decode work (16-bit
// caches of the query type; same pools, head shape and block size in both).
// The decode partials it leaves are merged by launch_decode_reduce(d).
hipError_t launch_mixed(const PrefillParams& pf, const DecodeParams& d, hipStream_t stream);
// Compute units of the current device.
int cu_count();
// Upper bound of the decode waves that can have work, from host-known sizes.
int64_t wave_work_bound(const DecodeParams& p);
// LDS bytes the prefill kernel needs (two stages of a K and a V tile).
size_t prefill_smem_bytes(int head_dim);
hipError_t launch_probe_read(const void* src, size_t bytes, void* sink, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

}  // namespace pa
