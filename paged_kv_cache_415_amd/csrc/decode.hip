// Paged decode attention on gfx950.
//
// What is computed (bogosort page "五十三：vLLM-PagedAttention" §8, ybb.press
// page "vLLM 与 LLM 推理部署实战" §2.3): for each sequence and query head, the
// query attends every cached token of the sequence, whose K/V are found
// block by block through the block table.
//
// Work decomposition: one workgroup of four wave64s per
// (sequence, KV head, partition of `partition` tokens).  The partition's
// slice of the block table is staged in LDS once; each wave then walks
// 32-token steps of the partition (steps w, w+4, ...), keeping its own
// online-softmax state (running max m, running sum l, unnormalised output).
// The four waves merge through LDS at the end.  A sequence with one
// partition gets its output written directly; longer sequences write
// partial (o, m, l) triples that lse_reduce_kernel merges.
//
// Matrix cores: all query heads of a KV group are the 16 columns of one
// MFMA tile (group <= 16; unused columns are zero queries), so each K/V
// byte loaded from HBM is used by every head of its group:
//   S^T[token][head] = K[token][:] . Q[head][:]     v_mfma_f32_16x16x32
//   O^T[dim][head]  += V^T[dim][token] P^T[token][head]
// Taking the transposed products makes the score tile's register layout
// (lane = head column, registers = 4 token rows per 16-lane group) exactly
// the B-operand layout the value product needs, so probabilities never
// move between lanes, and the running max/sum of a head live in that
// head's own lanes.  The value operand wants 4+4 tokens of one dimension
// per lane while the cache stores dimensions contiguously; each lane loads
// 16-byte row pieces and transposes them in registers with byte permutes.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<_Float16> {
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Dynamic LDS: block-table slice, per-wave (m, l) and per-wave outputs.
struct DecodeSmem {
  int* tab;
  float* m;   // [kWaves][16]
  float* l;   // [kWaves][16]
  float* o;   // [kWaves][group][D]
};

__device__ __forceinline__ DecodeSmem carve(char* base, int ntab, int group, int dim) {
  DecodeSmem s;
  s.tab = reinterpret_cast<int*>(base);
  int off = ((ntab * 4 + 15) / 16) * 16;
  s.m = reinterpret_cast<float*>(base + off);
  s.l = s.m + kWaves * 16;
  s.o = s.l + kWaves * 16;
  (void)group;
  (void)dim;
  return s;
}

size_t decode_smem_bytes(int partition, int block_size, int group, int dim) {
  const int ntab = (partition + block_size - 1) / block_size;
  return ((ntab * 4 + 15) / 16) * 16 + 2 * kWaves * 16 * 4 + (size_t)kWaves * group * dim * 4;
}

// Shared prologue: clamp the length, find this workgroup's token range and
// stage the block-table slice.  Returns false when the workgroup has no work.
struct Range {
  int len, start, end, nparts;
};

__device__ __forceinline__ bool decode_prologue(const DecodeParams& p, const DecodeSmem& sm,
                                                Range& r) {
  const int seq = blockIdx.z, part = blockIdx.x;
  int len = p.seq_lens[seq];
  len = len < p.max_len ? len : p.max_len;
  r.len = len;
  r.start = part * p.partition;
  r.nparts = len > 0 ? (len + p.partition - 1) / p.partition : 0;
  if (r.start >= len) return false;
  r.end = min(len, r.start + p.partition);
  const int nblk = (r.end - r.start + p.block_size - 1) / p.block_size;
  const int* row = p.block_tables + (int64_t)seq * p.max_blocks + r.start / p.block_size;
  for (int i = threadIdx.x; i < nblk; i += kThreads) sm.tab[i] = row[i];
  __syncthreads();
  return true;
}

// Zero output for sequences with no tokens (written once, by partition 0).
template <typename QT>
__device__ __forceinline__ void zero_output(const DecodeParams& p) {
  const int seq = blockIdx.z, kvh = blockIdx.y;
  QT* out = reinterpret_cast<QT*>(p.out) + ((int64_t)seq * p.num_q_heads + kvh * p.group) * p.head_dim;
  for (int i = threadIdx.x; i < p.group * p.head_dim; i += kThreads) out[i] = (QT)0.0f;
}

// Merge the four waves' states and write the output or the partials.
template <typename QT>
__device__ __forceinline__ void merge_and_store(const DecodeParams& p, const DecodeSmem& sm,
                                                const Range& r) {
  __syncthreads();
  const int seq = blockIdx.z, kvh = blockIdx.y, part = blockIdx.x;
  const int D = p.head_dim, g = p.group;
  for (int idx = threadIdx.x; idx < g * D; idx += kThreads) {
    const int j = idx / D, d = idx - j * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w * 16 + j]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.m[w * 16 + j];
      if (mw != -INFINITY) {       // idle waves left no state
        const float wt = __builtin_amdgcn_exp2f(mw - M);
        O += wt * sm.o[(w * g + j) * D + d];
        L += wt * sm.l[w * 16 + j];
      }
    }
    const int h = kvh * g + j;
    if (r.nparts == 1) {
      QT* out = reinterpret_cast<QT*>(p.out);
      out[((int64_t)seq * p.num_q_heads + h) * D + d] = (QT)(O / L * p.v_scale);
    } else {
      const int64_t b = ((int64_t)seq * p.num_q_heads + h) * p.max_parts + part;
      p.part_o[b * D + d] = O;
      if (d == 0) {
        p.part_m[b] = M;
        p.part_l[b] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA decode for 16-bit and fp8 caches.
//   QT: query / output / MFMA operand type (__bf16 or _Float16)
//   FP8: cache holds E4M3 codes (decoded exactly to QT)
// ---------------------------------------------------------------------------
template <typename QT, bool FP8, int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
  extern __shared__ __align__(16) char smem_raw[];
  constexpr int NC = D / 32;     // QK MFMAs per 16-token tile (K = 32 dims each)
  constexpr int DPL = D / 16;    // value dims per lane = PV MFMAs per 32-token step
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int VW = DPL * EB / 4;   // dwords per V row piece (1, 2 or 4)
  const DecodeSmem sm = carve(smem_raw, (p.partition + BS - 1) / BS, p.group, D);
  Range r;
  if (p.seq_lens[blockIdx.z] <= 0) {
    if (blockIdx.x == 0) zero_output<QT>(p);
    return;
  }
  if (!decode_prologue(p, sm, r)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = lane >> 4;      // 16-lane group: selects k-slots / token rows
  const int c16 = lane & 15;    // column (query head) or row (token / dim) index
  const int kvh = blockIdx.y, seq = blockIdx.z;
  const int g = p.group;

  // Query operand (B of S^T = K Q^T): head column c16, 8 dims per MFMA.
  // The dims a lane group covers in MFMA c follow the order in which K row
  // pieces are loaded (any permutation of the reduction index is allowed as
  // long as K and Q agree).
  u32x4 qop[NC];
  {
    const QT* qrow = reinterpret_cast<const QT*>(p.q) +
                     ((int64_t)seq * p.num_q_heads + kvh * g + c16) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = FP8 ? (64 * (c >> 1) + 16 * G + 8 * (c & 1)) : (32 * c + 8 * G);
      qop[c] = (c16 < g) ? ld16(qrow + d0) : u32x4{0, 0, 0, 0};
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[DPL];
#pragma unroll
  for (int n = 0; n < DPL; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntok = r.end - r.start;
  const int nsteps = (ntok + 31) >> 5;
  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);

  for (int t = wave; t < nsteps; t += kWaves) {
    const int rel0 = t * 32;                   // token offset of the step in the partition
    u32x4 ka[2][NC];
    uint32_t vw[2][4][VW];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int rel = rel0 + 16 * tau;
      if (rel < ntok) {
        const int blk = sm.tab[rel / BS];
        const int row0 = rel % BS;
        const int64_t tile = (((int64_t)blk * p.num_kv_heads + kvh) * BS + row0) * D;   // elements
        // K: this lane's token row c16
        const char* kt = kpool + (tile + (int64_t)c16 * D) * EB;
        if constexpr (FP8) {
#pragma unroll
          for (int h = 0; h < D / 64; ++h) {
            const u32x4 raw = ld16(kt + 64 * h + 16 * G);
            ka[tau][2 * h] = u32x4{fp8x2_to<QT>(raw.x, false), fp8x2_to<QT>(raw.x, true),
                                   fp8x2_to<QT>(raw.y, false), fp8x2_to<QT>(raw.y, true)};
            ka[tau][2 * h + 1] = u32x4{fp8x2_to<QT>(raw.z, false), fp8x2_to<QT>(raw.z, true),
                                       fp8x2_to<QT>(raw.w, false), fp8x2_to<QT>(raw.w, true)};
          }
        } else {
#pragma unroll
          for (int c = 0; c < NC; ++c) ka[tau][c] = ld16(kt + (32 * c + 8 * G) * 2);
        }
        // V: token rows 4G + i, dims DPL*c16 .. DPL*c16 + DPL - 1
        const char* vt = vpool + (tile + (int64_t)(4 * G) * D + DPL * c16) * EB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const char* src = vt + (int64_t)i * D * EB;
          if constexpr (VW == 4) {
            const u32x4 x = ld16(src);
            vw[tau][i][0] = x.x; vw[tau][i][1] = x.y; vw[tau][i][2] = x.z; vw[tau][i][3] = x.w;
          } else if constexpr (VW == 2) {
            const u32x2 x = ld8(src);
            vw[tau][i][0] = x.x; vw[tau][i][1] = x.y;
          } else {
            vw[tau][i][0] = ld4(src);
          }
        }
        // rows past the end hold stale or poisoned data: zero their values
        // (a zero probability does not cancel a NaN in the product)
        if (rel + 16 > ntok) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (rel + 4 * G + i >= ntok) {
#pragma unroll
              for (int w = 0; w < VW; ++w) vw[tau][i][w] = 0u;
            }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[tau][c] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int w = 0; w < VW; ++w) vw[tau][i][w] = 0u;
      }
    }

    // Scores: S^T tile tau, lane (G, c16) holds tokens 4G+i of head c16.
    float s[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sc = Mma<QT>::mma(ka[tau][c], qop[c], sc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rel = rel0 + 16 * tau + 4 * G + i;
        s[tau][i] = (rel < ntok) ? sc[i] * p.qk_scale_log2 : -INFINITY;
      }
    }
    float smax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    smax = xor_max(smax, 16);
    smax = xor_max(smax, 32);
    const float m_new = fmaxf(m_run, smax);     // finite: every step has a valid token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    uint32_t pw[4];
    float psum = 0.f;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float a = __builtin_amdgcn_exp2f(s[tau][i] - m_new);
        const float b = __builtin_amdgcn_exp2f(s[tau][i + 1] - m_new);
        const uint32_t w = pack2<QT>(a, b);
        pw[tau * 2 + i / 2] = w;
        // sum the rounded probabilities so that the weights stay normalised
        psum += lo_f32<QT>(w) + hi_f32<QT>(w);
      }
    }
    l_run = l_run * alpha + psum;
    const u32x4 pop = {pw[0], pw[1], pw[2], pw[3]};

    // Values: A operand for dim DPL*c16 + n holds tokens 4G+0..3 of tile 0
    // then 4G+0..3 of tile 1.
#pragma unroll
    for (int n = 0; n < DPL; ++n) {
      u32x4 a;
      if constexpr (FP8) {
        const int w = n >> 2, k = n & 3;
        uint32_t x[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const uint32_t r0 = vw[tau][0][w], r1 = vw[tau][1][w], r2 = vw[tau][2][w], r3 = vw[tau][3][w];
          const uint32_t ta = (k & 1) ? perm(r1, r0, 0x07030501u) : perm(r1, r0, 0x06020400u);
          const uint32_t tc = (k & 1) ? perm(r3, r2, 0x07030501u) : perm(r3, r2, 0x06020400u);
          x[tau] = (k & 2) ? perm(tc, ta, 0x07060302u) : perm(tc, ta, 0x05040100u);
        }
        a = u32x4{fp8x2_to<QT>(x[0], false), fp8x2_to<QT>(x[0], true),
                  fp8x2_to<QT>(x[1], false), fp8x2_to<QT>(x[1], true)};
      } else {
        const int w = n >> 1;
        const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
        a = u32x4{perm(vw[0][1][w], vw[0][0][w], sel), perm(vw[0][3][w], vw[0][2][w], sel),
                  perm(vw[1][1][w], vw[1][0][w], sel), perm(vw[1][3][w], vw[1][2][w], sel)};
      }
      acc[n] = acc[n] * alpha;
      acc[n] = Mma<QT>::mma(a, pop, acc[n]);
    }
  }

  // Wave state -> LDS.  lane (G, c16) holds head c16, dims DPL*(4G+i) + n.
  float l_tot = xor_sum(l_run, 16);
  l_tot = xor_sum(l_tot, 32);
  if (c16 < g) {
    if (G == 0) {
      sm.m[wave * 16 + c16] = m_run;
      sm.l[wave * 16 + c16] = l_tot;
    }
    float* o = sm.o + (wave * g + c16) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int n = 0; n < DPL; ++n) o[DPL * (4 * G + i) + n] = acc[n][i];
  }
  merge_and_store<QT>(p, sm, r);
}

// ---------------------------------------------------------------------------
// fp32 decode (VALU): the small fp32 workloads.  Same grid, partitions and
// merge as the MFMA kernel; each wave handles one token at a time with the
// head dimension spread over its lanes.
// ---------------------------------------------------------------------------
template <int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(DecodeParams p) {
  extern __shared__ __align__(16) char smem_raw[];
  constexpr int E = D / 64;
  const DecodeSmem sm = carve(smem_raw, (p.partition + BS - 1) / BS, p.group, D);
  Range r;
  if (p.seq_lens[blockIdx.z] <= 0) {
    if (blockIdx.x == 0) zero_output<float>(p);
    return;
  }
  if (!decode_prologue(p, sm, r)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kvh = blockIdx.y, seq = blockIdx.z, g = p.group;
  const float* q = reinterpret_cast<const float*>(p.q) + ((int64_t)seq * p.num_q_heads + kvh * g) * D;
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
  const float* kpool = reinterpret_cast<const float*>(p.k_pool);
  const float* vpool = reinterpret_cast<const float*>(p.v_pool);
  for (int tok = r.start + wave; tok < r.end; tok += kWaves) {
    const int rel = tok - r.start;
    const int blk = sm.tab[rel / BS];
    const int64_t rowoff = (((int64_t)blk * p.num_kv_heads + kvh) * BS + rel % BS) * D;
    float kv[E], vv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kv[e] = kpool[rowoff + lane + 64 * e];
      vv[e] = vpool[rowoff + lane + 64 * e];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < g) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot += qv[j][e] * kv[e];
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) dot = xor_sum(dot, msk);
        const float sc = dot * p.qk_scale_log2;
        const float m_new = fmaxf(m[j], sc);
        const float alpha = __builtin_amdgcn_exp2f(m[j] - m_new);
        const float pr = __builtin_amdgcn_exp2f(sc - m_new);
        l[j] = l[j] * alpha + pr;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[j][e] = acc[j][e] * alpha + pr * vv[e];
        m[j] = m_new;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < g) {
      if (lane == 0) {
        sm.m[wave * 16 + j] = m[j];
        sm.l[wave * 16 + j] = l[j];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) sm.o[(wave * g + j) * D + lane + 64 * e] = acc[j][e];
    }
  }
  merge_and_store<float>(p, sm, r);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split partials:
//   M = max_i m_i,  out = v_scale * sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i
// ---------------------------------------------------------------------------
template <typename QT>
__global__ __launch_bounds__(128) void lse_reduce_kernel(DecodeParams p) {
  const int h = blockIdx.x, seq = blockIdx.y;
  int len = p.seq_lens[seq];
  len = len < p.max_len ? len : p.max_len;
  if (len <= 0) return;
  const int nparts = (len + p.partition - 1) / p.partition;
  if (nparts <= 1) return;
  const int64_t b = ((int64_t)seq * p.num_q_heads + h) * p.max_parts;
  float M = -INFINITY;
  for (int i = 0; i < nparts; ++i) M = fmaxf(M, p.part_m[b + i]);
  float L = 0.f;
  for (int i = 0; i < nparts; ++i) L += __builtin_amdgcn_exp2f(p.part_m[b + i] - M) * p.part_l[b + i];
  const float inv = p.v_scale / L;
  QT* out = reinterpret_cast<QT*>(p.out) + ((int64_t)seq * p.num_q_heads + h) * p.head_dim;
  for (int d = threadIdx.x; d < p.head_dim; d += blockDim.x) {
    float O = 0.f;
    for (int i = 0; i < nparts; ++i)
      O += __builtin_amdgcn_exp2f(p.part_m[b + i] - M) * p.part_o[(b + i) * p.head_dim + d];
    out[d] = (QT)(O * inv);
  }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
template <typename QT, bool FP8, int D>
static void launch_mfma_bs(const DecodeParams& p, dim3 grid, size_t smem, hipStream_t s) {
  if (p.block_size == 16)
    hipLaunchKernelGGL((decode_mfma_kernel<QT, FP8, D, 16>), grid, dim3(kThreads), smem, s, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<QT, FP8, D, 32>), grid, dim3(kThreads), smem, s, p);
}

template <typename QT, bool FP8>
static void launch_mfma(const DecodeParams& p, dim3 grid, size_t smem, hipStream_t s) {
  if (p.head_dim == 128)
    launch_mfma_bs<QT, FP8, 128>(p, grid, smem, s);
  else
    launch_mfma_bs<QT, FP8, 64>(p, grid, smem, s);
}

hipError_t launch_decode_attention(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  const dim3 grid(p.max_parts, p.num_kv_heads, p.num_seqs);
  const size_t smem = decode_smem_bytes(p.partition, p.block_size, p.group, p.head_dim);
  if (p.cache_dtype == kF32) {
    if (p.head_dim == 128) {
      if (p.block_size == 16)
        hipLaunchKernelGGL((decode_f32_kernel<128, 16>), grid, dim3(kThreads), smem, stream, p);
      else
        hipLaunchKernelGGL((decode_f32_kernel<128, 32>), grid, dim3(kThreads), smem, stream, p);
    } else {
      if (p.block_size == 16)
        hipLaunchKernelGGL((decode_f32_kernel<64, 16>), grid, dim3(kThreads), smem, stream, p);
      else
        hipLaunchKernelGGL((decode_f32_kernel<64, 32>), grid, dim3(kThreads), smem, stream, p);
    }
  } else {
    const bool fp8 = p.cache_dtype == kFP8;
    if (p.q_dtype == kBF16) {
      if (fp8) launch_mfma<__bf16, true>(p, grid, smem, stream);
      else launch_mfma<__bf16, false>(p, grid, smem, stream);
    } else {
      if (fp8) launch_mfma<_Float16, true>(p, grid, smem, stream);
      else launch_mfma<_Float16, false>(p, grid, smem, stream);
    }
  }
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.max_parts <= 1) return hipSuccess;
  const dim3 grid(p.num_q_heads, p.num_seqs);
  if (p.q_dtype == kF32)
    hipLaunchKernelGGL(lse_reduce_kernel<float>, grid, dim3(128), 0, stream, p);
  else if (p.q_dtype == kBF16)
    hipLaunchKernelGGL(lse_reduce_kernel<__bf16>, grid, dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(lse_reduce_kernel<_Float16>, grid, dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
