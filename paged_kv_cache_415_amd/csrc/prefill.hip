// Causal prefill chunk over a paged context on gfx950.
//
// What is computed (bogosort page "五十三：vLLM-PagedAttention" §15 Chunked
// Prefill; ai-engineering page "推理引擎内部机制" section "分块预填充保护 TTFT
// 尾部"): a prompt is prefilled in chunks; chunk query i of a sequence with n
// context tokens and chunk length L sits at position n - L + i and attends
// keys 0 .. n - L + i, all read through the block table.
//
// Work decomposition: one workgroup (four wave64s) per (tile of query rows,
// KV head, sequence).  A tile holds 128 query rows = (128 / group)
// consecutive chunk positions x the group's query heads, so one staged K/V
// tile serves every head of the group.  The workgroup walks the context in
// 64-key tiles: the tile's rows are gathered through the LDS-cached block
// table into LDS with 16-byte loads, then each wave (32 query rows) forms
//   S^T[key][row] = K[key][:] . Q[row][:]            (v_mfma_f32_16x16x32)
//   O^T[dim][row] += V^T[dim][key] P^T[key][row]     (v_mfma_f32_16x16x32)
// with an online softmax per query row.  As in the decode kernel, the score
// tile's register layout is the value product's B operand, so
// probabilities stay in their lanes.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <typename T>
struct PMma;

template <>
struct PMma<__bf16> {
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct PMma<_Float16> {
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

constexpr int kPThreads = 256;
constexpr int kRowsPerWG = 128;
constexpr int kKeyTile = 64;

size_t prefill_smem_bytes(int head_dim, int max_blocks) {
  const int stride = head_dim + 8;  // padded row, in elements
  return (size_t)2 * kKeyTile * stride * 2 + (size_t)max_blocks * 4;
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(kPThreads) void prefill_mfma_kernel(PrefillParams p) {
  extern __shared__ __align__(16) char smem_raw[];
  constexpr int NC = D / 32;
  constexpr int DPL = D / 16;
  constexpr int STRIDE = D + 8;             // LDS row stride (elements): spreads banks
  constexpr int VPR = D / 8;                // 16-byte vectors per row
  T* k_lds = reinterpret_cast<T*>(smem_raw);
  T* v_lds = k_lds + kKeyTile * STRIDE;
  int* tab = reinterpret_cast<int*>(v_lds + kKeyTile * STRIDE);

  const int seq = blockIdx.z, kvh = blockIdx.y;
  const int g = p.group;
  const int qpos = kRowsPerWG / g;          // chunk positions per workgroup
  const int q0 = p.query_start_loc[seq];
  const int L = p.query_start_loc[seq + 1] - q0;
  const int p0 = blockIdx.x * qpos;
  if (p0 >= L) return;
  int n = p.seq_lens[seq];
  const int cap = p.max_blocks * BS;
  n = n < cap ? n : cap;
  if (n < L) return;                        // malformed: the chunk must be in the context
  const int ctx0 = n - L;                   // position of chunk query 0
  const int last_pos = min(p0 + qpos, L) - 1;
  const int kend = ctx0 + last_pos + 1;     // keys [0, kend) can be visible to this tile
  const int ntab = (kend + BS - 1) / BS;
  const int* trow = p.block_tables + (int64_t)seq * p.max_blocks;
  for (int i = threadIdx.x; i < ntab; i += kPThreads) tab[i] = trow[i];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = lane >> 4, c16 = lane & 15;

  // This lane's query row in each of the wave's two column tiles.
  int pos[2], head[2];
  bool valid[2];
  int lim[2];
  u32x4 qop[2][NC];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int rho = wave * 32 + b * 16 + c16;
    pos[b] = p0 + rho / g;
    head[b] = rho % g;
    valid[b] = pos[b] < L;
    lim[b] = valid[b] ? ctx0 + pos[b] : n - 1;     // last visible key
    const T* qrow = reinterpret_cast<const T*>(p.q) +
                    ((int64_t)(q0 + pos[b]) * p.num_q_heads + kvh * g + head[b]) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) qop[b][c] = valid[b] ? ld16(qrow + 32 * c + 8 * G) : u32x4{0, 0, 0, 0};
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 acc[2][DPL];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int nn = 0; nn < DPL; ++nn) acc[b][nn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);
  const int ntiles = (kend + kKeyTile - 1) / kKeyTile;
  __syncthreads();   // block-table slice visible

  for (int kt = 0; kt < ntiles; ++kt) {
    // ---- gather the 64-key K/V tile through the block table into LDS
#pragma unroll
    for (int it = 0; it < kKeyTile * VPR / kPThreads; ++it) {
      const int idx = it * kPThreads + threadIdx.x;
      const int row = idx / VPR, vec = idx % VPR;
      const int key = kt * kKeyTile + row;
      u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (key < kend) {
        const int blk = tab[key / BS];
        const int64_t off = ((((int64_t)blk * p.num_kv_heads + kvh) * BS + key % BS) * D + vec * 8) * 2;
        kx = ld16(kpool + off);
        vx = ld16(vpool + off);
      }
      st16(k_lds + row * STRIDE + vec * 8, kx);
      st16(v_lds + row * STRIDE + vec * 8, vx);
    }
    __syncthreads();

    // ---- scores for 4 key row-tiles x 2 query column-tiles
    float s[4][2][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x4 ka[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        ka[c] = *reinterpret_cast<const u32x4*>(k_lds + (16 * a + c16) * STRIDE + 32 * c + 8 * G);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) sc = PMma<T>::mma(ka[c], qop[b][c], sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt * kKeyTile + 16 * a + 4 * G + i;
          s[a][b][i] = (key <= lim[b]) ? mul_rn(sc[i], p.qk_scale_log2) : -INFINITY;
        }
      }
    }
    // ---- online softmax per query row (lane column), probabilities -> operands
    u32x4 pop[2][2];   // [key pair][column tile]
    float alpha[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float mx = -INFINITY;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[a][b][i]);
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const float m_new = fmaxf(m_run[b], mx);
      alpha[b] = __builtin_amdgcn_exp2f(m_run[b] - m_new);
      m_run[b] = m_new;
      float psum = 0.f;
      uint32_t w[4][2];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const uint32_t pw = pack2<T>(__builtin_amdgcn_exp2f(s[a][b][i] - m_new),
                                       __builtin_amdgcn_exp2f(s[a][b][i + 1] - m_new));
          w[a][i / 2] = pw;
          psum += lo_f32<T>(pw) + hi_f32<T>(pw);
        }
      l_run[b] = l_run[b] * alpha[b] + psum;
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
        pop[ap][b] = u32x4{w[2 * ap][0], w[2 * ap][1], w[2 * ap + 1][0], w[2 * ap + 1][1]};
#pragma unroll
      for (int nn = 0; nn < DPL; ++nn) acc[b][nn] = acc[b][nn] * alpha[b];
    }
    // ---- values: A operand rows = dims DPL*c16 + nn, k-slots = keys of a pair
#pragma unroll
    for (int ap = 0; ap < 2; ++ap) {
      uint32_t vr[2][4][DPL / 2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const T* src = v_lds + (16 * (2 * ap + half) + 4 * G + i) * STRIDE + DPL * c16;
          if constexpr (DPL == 8) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(src);
            vr[half][i][0] = x.x; vr[half][i][1] = x.y; vr[half][i][2] = x.z; vr[half][i][3] = x.w;
          } else {
            const u32x2 x = *reinterpret_cast<const u32x2*>(src);
            vr[half][i][0] = x.x; vr[half][i][1] = x.y;
          }
        }
#pragma unroll
      for (int nn = 0; nn < DPL; ++nn) {
        const int w = nn >> 1;
        const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
        const u32x4 va = {perm(vr[0][1][w], vr[0][0][w], sel), perm(vr[0][3][w], vr[0][2][w], sel),
                          perm(vr[1][1][w], vr[1][0][w], sel), perm(vr[1][3][w], vr[1][2][w], sel)};
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[b][nn] = PMma<T>::mma(va, pop[ap][b], acc[b][nn]);
      }
    }
    __syncthreads();   // tile consumed before the next gather overwrites it
  }

  // ---- normalise and store: lane (G, c16) holds dims DPL*(4G+i) + nn of its row
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float l = xor_sum(l_run[b], 16);
    l = xor_sum(l, 32);
    if (!valid[b]) continue;
    const float inv = p.v_scale / l;
    T* orow = reinterpret_cast<T*>(p.out) +
              ((int64_t)(q0 + pos[b]) * p.num_q_heads + kvh * g + head[b]) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[DPL / 2];
#pragma unroll
      for (int nn = 0; nn < DPL; nn += 2) w[nn / 2] = pack2<T>(acc[b][nn][i] * inv, acc[b][nn + 1][i] * inv);
      T* dst = orow + DPL * (4 * G + i);
      if constexpr (DPL == 8) {
        st16(dst, u32x4{w[0], w[1], w[2], w[3]});
      } else {
        *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
      }
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_q_len == 0) return hipSuccess;
  const int qpos = kRowsPerWG / p.group;
  const dim3 grid((p.max_q_len + qpos - 1) / qpos, p.num_kv_heads, p.num_seqs);
  const size_t smem = prefill_smem_bytes(p.head_dim, p.max_blocks);
#define PA_PREFILL(T, D, BS) \
  hipLaunchKernelGGL((prefill_mfma_kernel<T, D, BS>), grid, dim3(kPThreads), smem, stream, p)
  if (p.q_dtype == kBF16) {
    if (p.head_dim == 128) {
      if (p.block_size == 16) PA_PREFILL(__bf16, 128, 16); else PA_PREFILL(__bf16, 128, 32);
    } else {
      if (p.block_size == 16) PA_PREFILL(__bf16, 64, 16); else PA_PREFILL(__bf16, 64, 32);
    }
  } else {
    if (p.head_dim == 128) {
      if (p.block_size == 16) PA_PREFILL(_Float16, 128, 16); else PA_PREFILL(_Float16, 128, 32);
    } else {
      if (p.block_size == 16) PA_PREFILL(_Float16, 64, 16); else PA_PREFILL(_Float16, 64, 32);
    }
  }
#undef PA_PREFILL
  return hipGetLastError();
}

}  // namespace pa
