// Causal prefill chunk over a paged context on gfx950: the kernels and
// their launcher.  The 16-bit / fp8 tile program is in prefill_dev.h.
#include "prefill_dev.h"

namespace pa {

// Two stages of (K tile, V tile).
size_t prefill_smem_bytes(int head_dim) { return (size_t)2 * 2 * kKeyTile * head_dim * 2; }

template <typename T, int D, int BS, bool KV8 = false, bool I8 = false>
__global__ __launch_bounds__(kPThreads) void prefill_mfma_kernel(PrefillParams p) {
  int seq, kvh, qtile;
  prefill_work(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), gridDim.x * gridDim.y * gridDim.z,
               gridDim.x, gridDim.y, seq, kvh, qtile);
  prefill_tile<T, D, BS, KV8, I8>(p, seq, kvh, qtile);
}

// ---------------------------------------------------------------------------
// fp32 cache (small workloads, vector unit): one wave per (chunk position,
// KV head, sequence) computes the group's query heads.  The head dimension
// is spread over the lanes; keys 0 .. n - L + pos are taken one at a time
// from groups of 16 whose rows are loaded together, with an online softmax
// per head.
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillParams p) {
  constexpr int E = D / 64;
  constexpr int kGroup = 16;
  const int pos = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int q0 = p.query_start_loc[seq];
  const int L = p.query_start_loc[seq + 1] - q0;
  if (pos >= L) return;
  int n = p.seq_lens[seq];
  const int cap = p.max_blocks * BS;
  n = n < cap ? n : cap;
  if (n < L) return;                       // malformed: the chunk must be in the context
  const int t_end = n - L + pos + 1;       // keys [0, t_end) are visible
  const int lane = threadIdx.x;
  const int g = p.group;
  const int* trow = p.block_tables + (int64_t)seq * p.max_blocks;
  const float* q = reinterpret_cast<const float*>(p.q) + ((int64_t)(q0 + pos) * p.num_q_heads + kvh * g) * D;
  const float* kpool = reinterpret_cast<const float*>(p.k_pool);
  const float* vpool = reinterpret_cast<const float*>(p.v_pool);
  float qv[16][E], acc[16][E], m[16], l[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      qv[j][e] = (j < g) ? q[j * D + lane + 64 * e] : 0.f;
      acc[j][e] = 0.f;
    }
  }
  for (int t0 = 0; t0 < t_end; t0 += kGroup) {
    float kv[kGroup][E], vv[kGroup][E];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int t = min(t0 + k, t_end - 1);   // past the end: the last key again (unused)
      const int64_t rowoff = (((int64_t)trow[t / BS] * p.num_kv_heads + kvh) * BS + t % BS) * D;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kv[k][e] = kpool[rowoff + lane + 64 * e];
        vv[k][e] = vpool[rowoff + lane + 64 * e];
      }
    }
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j < g && t0 + k < t_end) {
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) dot += qv[j][e] * kv[k][e];
#pragma unroll
          for (int msk = 32; msk >= 1; msk >>= 1) dot += __shfl_xor(dot, msk, 64);
          const float sc = mul_rn(dot, p.qk_scale_log2);
          const float m_new = fmaxf(m[j], sc);
          const float alpha = __builtin_amdgcn_exp2f(m[j] - m_new);
          const float pr = __builtin_amdgcn_exp2f(sc - m_new);
          l[j] = l[j] * alpha + pr;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[j][e] = acc[j][e] * alpha + pr * vv[k][e];
          m[j] = m_new;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < g) {
      float* orow = reinterpret_cast<float*>(p.out) + ((int64_t)(q0 + pos) * p.num_q_heads + kvh * g + j) * D;
      const float inv = p.v_scale / l[j];
#pragma unroll
      for (int e = 0; e < E; ++e) orow[lane + 64 * e] = acc[j][e] * inv;
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_q_len == 0) return hipSuccess;
  if (p.q_dtype == kF32) {
    const dim3 grid(p.max_q_len, p.num_kv_heads, p.num_seqs);
#define PA_PREFILL32(D, BS) hipLaunchKernelGGL((prefill_f32_kernel<D, BS>), grid, dim3(64), 0, stream, p)
#define PA_PREFILL32_BS(D)                       \
  switch (p.block_size) {                        \
    case 8: PA_PREFILL32(D, 8); break;           \
    case 16: PA_PREFILL32(D, 16); break;         \
    case 32: PA_PREFILL32(D, 32); break;         \
    default: PA_PREFILL32(D, 64); break;         \
  }
    if (p.head_dim == 128) { PA_PREFILL32_BS(128) } else { PA_PREFILL32_BS(64) }
#undef PA_PREFILL32_BS
#undef PA_PREFILL32
    return hipGetLastError();
  }
  const int qpos = kRowsPerWG / p.group;
  const dim3 grid((p.max_q_len + qpos - 1) / qpos, p.num_kv_heads, p.num_seqs);
  const size_t smem = prefill_smem_bytes(p.head_dim);
  const bool kv8 = p.cache_dtype == kFP8, i8 = p.cache_dtype == kI8;
#define PA_PREFILL(T, D, BS)                                                                          \
  do {                                                                                               \
    if (kv8) hipLaunchKernelGGL((prefill_mfma_kernel<T, D, BS, true>), grid, dim3(kPThreads), smem, stream, p); \
    else if (i8) hipLaunchKernelGGL((prefill_mfma_kernel<T, D, BS, true, true>), grid, dim3(kPThreads), smem, stream, p); \
    else hipLaunchKernelGGL((prefill_mfma_kernel<T, D, BS, false>), grid, dim3(kPThreads), smem, stream, p); \
  } while (0)
#define PA_PREFILL_BS(T, D)                      \
  switch (p.block_size) {                        \
    case 8: PA_PREFILL(T, D, 8); break;          \
    case 16: PA_PREFILL(T, D, 16); break;        \
    case 32: PA_PREFILL(T, D, 32); break;        \
    default: PA_PREFILL(T, D, 64); break;        \
  }
  if (p.q_dtype == kBF16) {
    if (p.head_dim == 128) { PA_PREFILL_BS(__bf16, 128) } else { PA_PREFILL_BS(__bf16, 64) }
  } else {
    if (p.head_dim == 128) { PA_PREFILL_BS(_Float16, 128) } else { PA_PREFILL_BS(_Float16, 64) }
  }
#undef PA_PREFILL_BS
#undef PA_PREFILL
  return hipGetLastError();
}

}  // namespace pa
