// Slot scatter (reshape_and_cache), block copies (whole-block and
// partial-block copy-on-write, one layer or many), block moves between pools
// (swapping to host memory) and the HBM probe kernels.
//
// The scatter follows the datawhalechina page "17. vLLM PagedAttention"
// (Step 3 item 3 / Step 4: each generated token's K/V goes into the
// physical block handed out for it) with the slot linearisation
// physical * block_size + offset.  The block copy follows the ybb.press page
// "vLLM 与 LLM 推理部署实战" §2.2 (a write to a shared block duplicates the
// whole block first).  Both are data movement: 16-byte loads and stores per
// thread, coalesced along head_dim; the quantising scatters (fp8 E4M3 with
// per-tensor scales, int8 with per-(block, KV head) scales) turn 16 source
// elements into one 16-byte store of codes.
#include <algorithm>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// One workgroup per token; threads walk the token's Hkv * D elements in
// 16-byte source vectors.  Same-type copy.
template <typename ElemBytesTag>
__global__ __launch_bounds__(256) void scatter_copy_kernel(ScatterParams p) {
  const int t = blockIdx.x;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0) return;
  const int64_t blk = slot / p.block_size;
  const int row = (int)(slot - blk * p.block_size);
  const int eb = p.src_elem_bytes;
  const int vec_per_head = p.head_dim * eb / 16;
  const int nvec = p.num_kv_heads * vec_per_head;
  const char* ksrc = (const char*)p.key + (int64_t)t * p.key_stride * eb;
  const char* vsrc = (const char*)p.value + (int64_t)t * p.value_stride * eb;
  for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
    const int h = i / vec_per_head;
    const int c = i - h * vec_per_head;
    const int64_t dst = (((blk * p.num_kv_heads + h) * p.block_size + row) * p.head_dim) * eb + c * 16;
    const int64_t src = (int64_t)h * p.head_dim * eb + c * 16;
    st16((char*)p.k_pool + dst, ld16(ksrc + src));
    st16((char*)p.v_pool + dst, ld16(vsrc + src));
  }
}

template <typename SrcT>
__device__ __forceinline__ float src_elem(const char* base, int i) {
  return (float)reinterpret_cast<const SrcT*>(base)[i];
}

// Quantising scatter into an fp8 E4M3 pool: each thread turns 4 source
// elements into 4 codes (one 32-bit store).  With VQ false only K is
// quantised and the V elements are copied unchanged (fp8 K cache beside a
// 16-bit V cache).
template <typename SrcT, bool VQ>
__global__ __launch_bounds__(256) void scatter_fp8_kernel(ScatterParams p) {
  const int t = blockIdx.x;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0) return;
  const int64_t blk = slot / p.block_size;
  const int row = (int)(slot - blk * p.block_size);
  // one thread per 4 elements of a head row (a 32-bit word of codes): the
  // per-element divides of a token are spread over the whole workgroup
  const int groups_per_head = p.head_dim / 4;
  const int ngroups = p.num_kv_heads * groups_per_head;
  const SrcT* ksrc = reinterpret_cast<const SrcT*>(p.key) + (int64_t)t * p.key_stride;
  const SrcT* vsrc = reinterpret_cast<const SrcT*>(p.value) + (int64_t)t * p.value_stride;
  for (int i = threadIdx.x; i < ngroups; i += blockDim.x) {
    const int h = i / groups_per_head;
    const int c = i - h * groups_per_head;
    const int64_t dst = ((blk * p.num_kv_heads + h) * p.block_size + row) * p.head_dim + c * 4;
    const int64_t src = (int64_t)h * p.head_dim + c * 4;
    if constexpr (!VQ) {
      const char* vs = reinterpret_cast<const char*>(vsrc + src);
      char* vd = (char*)p.v_pool + dst * (int64_t)sizeof(SrcT);
      if constexpr (sizeof(SrcT) == 2) *reinterpret_cast<u32x2*>(vd) = ld8(vs);
      else st16(vd, ld16(vs));
    }
#pragma unroll
    for (int which = 0; which < (VQ ? 2 : 1); ++which) {
      const SrcT* s = which ? vsrc : ksrc;
      const float scale = which ? p.v_scale : p.k_scale;
      uint32_t acc = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float x = (float)s[src + b];
        acc |= e4m3_encode(x / scale) << (8 * b);   // correctly rounded fp32 divide
      }
      *reinterpret_cast<uint32_t*>((char*)(which ? p.v_pool : p.k_pool) + dst) = acc;
    }
  }
}

// Quantising scatter into an int8 pool with one scale per (block, KV head):
// each thread turns 4 source elements of K and of V into 4 codes each.
template <typename SrcT>
__global__ __launch_bounds__(256) void scatter_i8_kernel(ScatterParams p) {
  const int t = blockIdx.x;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0) return;
  const int64_t blk = slot / p.block_size;
  const int row = (int)(slot - blk * p.block_size);
  const int groups_per_head = p.head_dim / 4;
  const int ngroups = p.num_kv_heads * groups_per_head;
  const SrcT* ksrc = reinterpret_cast<const SrcT*>(p.key) + (int64_t)t * p.key_stride;
  const SrcT* vsrc = reinterpret_cast<const SrcT*>(p.value) + (int64_t)t * p.value_stride;
  for (int i = threadIdx.x; i < ngroups; i += blockDim.x) {
    const int h = i / groups_per_head;
    const int c = i - h * groups_per_head;
    const int64_t dst = ((blk * p.num_kv_heads + h) * p.block_size + row) * p.head_dim + c * 4;
    const int64_t src = (int64_t)h * p.head_dim + c * 4;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const SrcT* s = which ? vsrc : ksrc;
      const float scale = (which ? p.v_scales : p.k_scales)[blk * p.num_kv_heads + h];
      uint32_t acc = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc |= ((uint32_t)i8_encode((float)s[src + b], scale) & 0xFFu) << (8 * b);
      *reinterpret_cast<uint32_t*>((char*)(which ? p.v_pool : p.k_pool) + dst) = acc;
    }
  }
}

// Copy nvec 16-byte vectors with the workgroups of grid dimension x; each
// thread keeps four loads in flight.
__device__ __forceinline__ void copy_vecs(char* dst, const char* src, int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const u32x4 a = ld16(src + i * 16), b = ld16(src + (i + stride) * 16);
    const u32x4 c = ld16(src + (i + 2 * stride) * 16), d = ld16(src + (i + 3 * stride) * 16);
    st16(dst + i * 16, a);
    st16(dst + (i + stride) * 16, b);
    st16(dst + (i + 2 * stride) * 16, c);
    st16(dst + (i + 3 * stride) * 16, d);
  }
  for (; i < nvec; i += stride) st16(dst + i * 16, ld16(src + i * 16));
}

// Workgroups along x for a copy of nvec vectors: four vectors per thread.
inline int copy_chunks(int64_t nvec) {
  int64_t c = (nvec + 1023) / 1024;
  return (int)(c < 1 ? 1 : (c > 64 ? 64 : c));
}

// One workgroup per (pair, chunk of the block); K and V pools both copied.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
  const int pair = blockIdx.y;
  const int64_t src = p.pairs[2 * pair];
  const int64_t dst = p.pairs[2 * pair + 1];
  const int64_t nvec = p.block_bytes / 16;
  char* k = static_cast<char*>(p.k_pool);
  char* v = static_cast<char*>(p.v_pool);
  copy_vecs(k + dst * p.block_bytes, k + src * p.block_bytes, nvec);
  copy_vecs(v + dst * p.block_bytes, v + src * p.block_bytes, nvec);
}

// Copy-on-write of a partly filled block (bogosort page "五十三：
// vLLM-PagedAttention" §17 Parallel Sampling: after a fork each sequence
// writes into its own blocks): only the rows [0, n) that hold tokens are
// copied, head by head (each head's rows are contiguous in a block).  n is
// clamped to [0, block_size].
__global__ __launch_bounds__(256) void copy_rows_kernel(CopyRowsParams p) {
  const int pair = blockIdx.y;
  const int64_t src = p.triples[3 * pair];
  const int64_t dst = p.triples[3 * pair + 1];
  int64_t n = p.triples[3 * pair + 2];
  n = n < 0 ? 0 : (n > p.block_size ? p.block_size : n);
  const int64_t head_bytes = (int64_t)p.block_size * p.row_bytes;
  const int64_t vph = n * p.row_bytes / 16;            // 16-byte vectors per head
  const int64_t nvec = vph * p.num_kv_heads;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t h = i / vph, v = i - h * vph;
    const int64_t so = (src * p.num_kv_heads + h) * head_bytes + v * 16;
    const int64_t d = (dst * p.num_kv_heads + h) * head_bytes + v * 16;
    st16((char*)p.k_pool + d, ld16((const char*)p.k_pool + so));
    st16((char*)p.v_pool + d, ld16((const char*)p.v_pool + so));
  }
}

// The same whole-block copies in the pools of every layer (one launch for a
// fork across the model: ybb.press page §2.2 Copy-on-Write 与共享前缀).
__global__ __launch_bounds__(256) void copy_layers_kernel(CopyLayersParams p) {
  const int pair = blockIdx.y, layer = blockIdx.z;
  const int64_t src = p.pairs[2 * pair];
  const int64_t dst = p.pairs[2 * pair + 1];
  char* k = static_cast<char*>(p.k_pools[layer]);
  char* v = static_cast<char*>(p.v_pools[layer]);
  const int64_t nvec = p.block_bytes / 16;
  copy_vecs(k + dst * p.block_bytes, k + src * p.block_bytes, nvec);
  copy_vecs(v + dst * p.block_bytes, v + src * p.block_bytes, nvec);
}

// Block moves between two pools (ybb.press page §三, the preemption bullet:
// blocks are swapped out to CPU memory and back).  Host memory is reached
// through its device mapping, so one launch moves any set of blocks.
__global__ __launch_bounds__(256) void swap_blocks_kernel(SwapParams p) {
  const int pair = blockIdx.y;
  const int64_t src = p.pairs[2 * pair];
  const int64_t dst = p.pairs[2 * pair + 1];
  copy_vecs(static_cast<char*>(p.dst) + dst * p.block_bytes,
            static_cast<const char*>(p.src) + src * p.block_bytes, p.block_bytes / 16);
}

hipError_t launch_scatter(const ScatterParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  dim3 grid(p.num_tokens), block(256);
  const bool vq = p.v_cache_dtype != p.src_dtype;   // V quantised too
  if (p.cache_dtype == kI8) {
    if (p.src_dtype == kBF16) hipLaunchKernelGGL(scatter_i8_kernel<__bf16>, grid, block, 0, stream, p);
    else if (p.src_dtype == kF16) hipLaunchKernelGGL(scatter_i8_kernel<_Float16>, grid, block, 0, stream, p);
    else hipLaunchKernelGGL(scatter_i8_kernel<float>, grid, block, 0, stream, p);
  } else if (p.cache_dtype == p.src_dtype) {
    hipLaunchKernelGGL(scatter_copy_kernel<void>, grid, block, 0, stream, p);
  } else if (p.src_dtype == kBF16) {
    if (vq) hipLaunchKernelGGL((scatter_fp8_kernel<__bf16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((scatter_fp8_kernel<__bf16, false>), grid, block, 0, stream, p);
  } else if (p.src_dtype == kF16) {
    if (vq) hipLaunchKernelGGL((scatter_fp8_kernel<_Float16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((scatter_fp8_kernel<_Float16, false>), grid, block, 0, stream, p);
  } else {
    if (vq) hipLaunchKernelGGL((scatter_fp8_kernel<float, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((scatter_fp8_kernel<float, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  dim3 grid(copy_chunks(p.block_bytes / 16), p.num_pairs), block(256);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyRowsParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  const int64_t nvec = (int64_t)p.num_kv_heads * p.block_size * p.row_bytes / 16;
  int chunks = (int)((nvec + 255) / 256);
  if (chunks > 64) chunks = 64;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(chunks, p.num_pairs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_copy_layers(const CopyLayersParams& p, hipStream_t stream) {
  if (p.num_pairs == 0 || p.num_layers == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_layers_kernel, dim3(copy_chunks(p.block_bytes / 16), p.num_pairs, p.num_layers),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const SwapParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(copy_chunks(p.block_bytes / 16), p.num_pairs), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- probes

// Grid-stride streaming read with non-temporal 16-byte loads (the fastest of
// the plain read kernels tried on MI355X: about 7.0 TB/s over 4 GiB with 2048
// workgroups of 256 threads, against 6.3 TB/s for ordinary loads).
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* src, int64_t nvec, u32x4* sink) {
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    acc ^= ld16_nt(src + i);
  }
  // fold the wave's values so the loads stay live; one store per workgroup
  for (int m = 32; m >= 1; m >>= 1) {
    acc.x ^= __shfl_xor(acc.x, m, 64);
    acc.y ^= __shfl_xor(acc.y, m, 64);
    acc.z ^= __shfl_xor(acc.z, m, 64);
    acc.w ^= __shfl_xor(acc.w, m, 64);
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(u32x4* dst, const u32x4* src, int64_t nvec) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    dst[i] = src[i];
  }
}

hipError_t launch_probe_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  const int64_t nvec = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(256), 0, stream,
                     (const u32x4*)src, nvec, (u32x4*)sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t nvec = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(256), 0, stream, (u32x4*)dst,
                     (const u32x4*)src, nvec);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Index checks: device-resident block ids, lengths, chunk offsets and slots
// compared against the sizes the caller states; nothing they name is read.
// err[0] = OR of the flags found, err[1] = number of bad sequences (tables)
// or tokens (slots), err[2] = the smallest bad sequence / token index.
// ---------------------------------------------------------------------------
__global__ void check_reset_kernel(int* err) {
  err[0] = 0;
  err[1] = 0;
  err[2] = 0x7FFFFFFF;
}

__global__ __launch_bounds__(256) void check_tables_kernel(CheckParams p) {
  __shared__ int flags_s;
  for (int s = blockIdx.x; s < p.num_items; s += gridDim.x) {
    if (threadIdx.x == 0) flags_s = 0;
    __syncthreads();
    const int n = p.seq_lens[s];
    const long long cap = (long long)p.max_blocks * p.block_size;
    int flags = 0;
    if (n < 0 || n > cap || (p.max_len > 0 && n > p.max_len)) flags |= kCheckLength;
    if (p.query_start_loc != nullptr && threadIdx.x == 0) {
      const int a = p.query_start_loc[s], b = p.query_start_loc[s + 1];
      if (a < 0 || b < a || b - a > n || (s + 1 == p.num_items && b != p.total)) flags |= kCheckChunk;
    }
    const int valid = n < 0 ? 0 : (int)(n > cap ? cap : n);
    const int nb = (valid + p.block_size - 1) / p.block_size;
    const int* row = p.block_tables + (int64_t)s * p.max_blocks;
    for (int b = threadIdx.x; b < nb; b += blockDim.x) {
      const int id = row[b];
      if (id < 0 || id >= p.num_blocks) flags |= kCheckBlockId;
    }
    if (flags) atomicOr(&flags_s, flags);
    __syncthreads();
    if (threadIdx.x == 0 && flags_s) {
      atomicOr(p.err, flags_s);
      atomicAdd(p.err + 1, 1);
      atomicMin(p.err + 2, s);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void check_slots_kernel(CheckParams p) {
  const int64_t limit = (int64_t)p.num_blocks * p.block_size;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < p.num_items; t += gridDim.x * blockDim.x) {
    if (p.slots[t] >= limit) {
      atomicOr(p.err, kCheckSlot);
      atomicAdd(p.err + 1, 1);
      atomicMin(p.err + 2, t);
    }
  }
}

hipError_t launch_check(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_reset_kernel, dim3(1), dim3(1), 0, stream, p.err);
  if (p.num_items > 0) {
    if (p.slots != nullptr) {
      const int grid = (int)std::min<int64_t>(1024, ((int64_t)p.num_items + 255) / 256);
      hipLaunchKernelGGL(check_slots_kernel, dim3(grid), dim3(256), 0, stream, p);
    } else {
      hipLaunchKernelGGL(check_tables_kernel, dim3(std::min(p.num_items, 4096)), dim3(256), 0, stream, p);
    }
  }
  return hipGetLastError();
}

}  // namespace pa
