// Causal prefill chunk over a paged context on gfx950.
//
// What is computed (bogosort page "五十三：vLLM-PagedAttention" §15 Chunked
// Prefill; ai-engineering page "推理引擎内部机制" section "分块预填充保护 TTFT
// 尾部"): a prompt is prefilled in chunks; chunk query i of a sequence with n
// context tokens and chunk length L sits at position n - L + i and attends
// keys 0 .. n - L + i, all read through the block table.
//
// Work decomposition: one workgroup (four wave64s) per (tile of query rows,
// KV head, sequence), mapped so that all query tiles of one (sequence, KV
// head) run on one XCD.  A tile holds 128 query rows = (128 / group)
// consecutive chunk positions x the group's query heads, so one staged K/V
// tile serves every head of the group.  The workgroup walks the context in
// 64-key tiles: the tile's rows are gathered through the LDS-cached block
// table with 16-byte loads (the next tile's loads are in flight while the
// current one is computed) and stored to LDS, then each wave (32 query rows)
// forms
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
constexpr float kSlack = 8.0f;   // log2 units
constexpr int kXcds = 8;
// Column of key k (0..63) of a tile in the transposed V tile: the key index
// [ap:1][h:1][G:2][i:2] becomes [ap][G][h][i], so that the keys a lane holds
// in the probability operand (tiles 2ap and 2ap+1, rows 4G + i) are adjacent.
__device__ __forceinline__ int vt_col(int k) {
  return (k & 0x20) | ((k & 0x0C) << 1) | ((k & 0x10) >> 2) | (k & 3);
}

// Byte offset of (dimension d, column col) in the transposed V tile: rows of
// 64 keys (128 B), taken in pairs as 256-byte lines whose sixteen 16-byte
// chunks are XOR-swizzled by d / (D/16), so that the 16 lanes reading one
// operand (dimensions (D/16) * c16 + nn) hit 16 different chunks.
template <int D>
__device__ __forceinline__ int vt_offset(int d, int col) {
  const int swz = (d / (D / 16)) & 15;
  const int chunk = (((d & 1) << 3) | (col >> 3)) ^ swz;
  return (d >> 1) * 256 + chunk * 16 + (col & 7) * 2;
}

template <typename T> constexpr uint32_t kOnes = 0;                  // two 1.0 values
template <> constexpr uint32_t kOnes<__bf16> = 0x3F803F80u;
template <> constexpr uint32_t kOnes<_Float16> = 0x3C003C00u;         // MI355X: 8 XCDs, workgroups dispatched round-robin

size_t prefill_smem_bytes(int head_dim, int max_blocks) {
  const int stride = head_dim + 8;  // padded K row, in elements
  return (size_t)kKeyTile * stride * 2 + (size_t)head_dim * kKeyTile * 2 + (size_t)max_blocks * 4;
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(kPThreads) void prefill_mfma_kernel(PrefillParams p) {
  extern __shared__ __align__(16) char smem_raw[];
  constexpr int NC = D / 32;
  constexpr int DPL = D / 16;
  constexpr int STRIDE = D + 8;             // K row stride in LDS (elements): spreads banks
  constexpr int VPR = D / 8;                // 16-byte vectors per row
  constexpr int KPT = kKeyTile * VPR / kPThreads;   // keys per thread in a tile's gather
  T* k_lds = reinterpret_cast<T*>(smem_raw);
  char* vt_lds = reinterpret_cast<char*>(k_lds + kKeyTile * STRIDE);   // V^T, D x 64 keys
  int* tab = reinterpret_cast<int*>(vt_lds + D * kKeyTile * 2);

  // Workgroup `lin` runs on XCD lin % kXcds.  Each XCD gets a contiguous
  // range of work items (query tile fastest), so the query tiles that read
  // one (sequence, KV head) context run on the same XCD and share its L2.
  const int nwg = gridDim.x * gridDim.y * gridDim.z;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int xq = nwg / kXcds, xr = nwg % kXcds;
  const int xcd = lin % kXcds, slot = lin / kXcds;
  const int work = xcd * xq + min(xcd, xr) + slot;   // a bijection of [0, nwg)
  const int qtile = work % gridDim.x;
  const int kvh = (work / gridDim.x) % gridDim.y;
  const int seq = work / (gridDim.x * gridDim.y);
  const int g = p.group;
  const int qpos = kRowsPerWG / g;          // chunk positions per workgroup
  const int q0 = p.query_start_loc[seq];
  const int L = p.query_start_loc[seq + 1] - q0;
  const int p0 = qtile * qpos;
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
  // logit = c * (q . k) with c = scale * k_scale * log2(e); a negative c is
  // applied as |c| with q negated, so maxima of raw products are maxima of
  // logits
  // (a zero scale runs as the smallest normal float, which rounds every
  // logit to 0 just the same but keeps -inf * scale = -inf for masked keys)
  const bool neg = p.qk_scale_log2 < 0.f;
  const float cscale = fmaxf(neg ? -p.qk_scale_log2 : p.qk_scale_log2, 1.17549435e-38f);

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
    for (int c = 0; c < NC; ++c) {
      qop[b][c] = valid[b] ? ld16(qrow + 32 * c + 8 * G) : u32x4{0, 0, 0, 0};
      if (neg) qop[b][c] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }
  }

  // Running max (in logit units, log2 domain), unnormalised outputs, and the
  // row sums of the rounded probabilities, formed on the matrix cores by a
  // value product against an all-ones operand (every row of acc_l holds the
  // column's sum).
  float m_run[2] = {-INFINITY, -INFINITY};
  f32x4 acc[2][DPL], acc_l[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    acc_l[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nn = 0; nn < DPL; ++nn) acc[b][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4 ones = {kOnes<T>, kOnes<T>, kOnes<T>, kOnes<T>};
  // first tile that needs the causal mask: every row sees keys <= ctx0 + p0
  const int min_lim = ctx0 + p0;

  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);
  const int ntiles = (kend + kKeyTile - 1) / kKeyTile;
  __syncthreads();   // block-table slice visible

  // The next tile's K/V rows are fetched into registers while the current
  // tile is computed; they go to LDS between two barriers.  Thread t loads
  // the 16-byte piece `vec` of KPT consecutive keys (a 16-lane group reads a
  // whole 256-byte row).  K is stored row-major; V is stored transposed (one
  // LDS row per dimension) with its keys permuted by vt_col, in the order in
  // which the probability operand holds them, so a lane's eight keys of one
  // dimension are 16 contiguous bytes (one ds_read_b128, no byte permutes).
  const int g_vec = threadIdx.x % VPR, g_kq = threadIdx.x / VPR;
  u32x4 kx[KPT], vx[KPT];
  auto gather = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = kt * kKeyTile + g_kq * KPT + i;
      kx[i] = u32x4{0, 0, 0, 0};
      vx[i] = u32x4{0, 0, 0, 0};
      if (key < kend) {
        const int blk = tab[key / BS];
        const int64_t off = ((((int64_t)blk * p.num_kv_heads + kvh) * BS + key % BS) * D + g_vec * 8) * 2;
        kx[i] = ld16(kpool + off);
        vx[i] = ld16(vpool + off);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) st16(k_lds + (g_kq * KPT + i) * STRIDE + g_vec * 8, kx[i]);
    // transpose KPT keys x 8 dims into 8 dims x KPT keys (16-bit lanes)
    const int col = vt_col(g_kq * KPT);     // KPT consecutive keys stay consecutive
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = g_vec * 8 + e;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      char* dst = vt_lds + vt_offset<D>(d, col);
      if constexpr (KPT == 4) {
        const uint32_t w0 = perm(vx[1][e >> 1], vx[0][e >> 1], sel);
        const uint32_t w1 = perm(vx[3][e >> 1], vx[2][e >> 1], sel);
        *reinterpret_cast<u32x2*>(dst) = u32x2{w0, w1};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = perm(vx[1][e >> 1], vx[0][e >> 1], sel);
      }
    }
  };
  gather(0);
  stash();
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const bool more = kt + 1 < ntiles;     // uniform over the workgroup
    if (more) gather(kt + 1);

    // ---- raw products q.k for 4 key row-tiles x 2 query column-tiles
    const bool diag = kt * kKeyTile + kKeyTile - 1 > min_lim;   // uniform
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
        for (int i = 0; i < 4; ++i) s[a][b][i] = sc[i];
      }
    }
    if (diag) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kt * kKeyTile + 16 * a + 4 * G + i > lim[b]) s[a][b][i] = -INFINITY;
    }
    // ---- online softmax per query row (lane column), probabilities -> operands
    u32x4 pop[2][2];   // [key pair][column tile]
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float mx = fmaxf(fmaxf(fmaxf(s[0][b][0], s[0][b][1]), fmaxf(s[0][b][2], s[0][b][3])),
                       fmaxf(fmaxf(s[1][b][0], s[1][b][1]), fmaxf(s[1][b][2], s[1][b][3])));
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[2][b][0], s[2][b][1]), fmaxf(s[2][b][2], s[2][b][3])),
                           fmaxf(fmaxf(s[3][b][0], s[3][b][1]), fmaxf(s[3][b][2], s[3][b][3]))));
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      mx *= cscale;   // cscale > 0: -inf stays -inf
      // Lazy rescaling (as in decode): the reference max moves only when a
      // row's max exceeds it by more than kSlack, so p <= 2^kSlack.  A row
      // whose keys are all masked in this tile has mx = -inf and keeps it.
      if (__builtin_amdgcn_ballot_w64(mx > m_run[b] + kSlack) != 0) {
        const float m_new = fmaxf(m_run[b], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_new);
        m_run[b] = m_new;
        acc_l[b] = acc_l[b] * alpha;
#pragma unroll
        for (int nn = 0; nn < DPL; ++nn) acc[b][nn] = acc[b][nn] * alpha;
      }
      // p = 2^(c * (q.k) - m): one fused multiply-add per score
      const float nm = -m_run[b];
      uint32_t w[4][2];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; i += 2)
          w[a][i / 2] = pack2<T>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[a][b][i], cscale, nm)),
                                 __builtin_amdgcn_exp2f(__builtin_fmaf(s[a][b][i + 1], cscale, nm)));
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
        pop[ap][b] = u32x4{w[2 * ap][0], w[2 * ap][1], w[2 * ap + 1][0], w[2 * ap + 1][1]};
    }
    // ---- values: A operand rows = dims DPL*c16 + nn, k-slots = the lane's
    // eight keys (keys 32ap + 4G + 0..3 and 32ap + 16 + 4G + 0..3), which
    // V^T holds contiguously at columns 32ap + 8G .. 32ap + 8G + 7
#pragma unroll
    for (int ap = 0; ap < 2; ++ap) {
#pragma unroll
      for (int nn = 0; nn < DPL; ++nn) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(
            vt_lds + vt_offset<D>(DPL * c16 + nn, 32 * ap + 8 * G));
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[b][nn] = PMma<T>::mma(va, pop[ap][b], acc[b][nn]);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) acc_l[b] = PMma<T>::mma(ones, pop[ap][b], acc_l[b]);
    }
    if (more) {
      __syncthreads();   // every wave is done with this tile
      stash();
      __syncthreads();   // the next tile is visible
    }
  }

  // ---- normalise and store: lane (G, c16) holds dims DPL*(4G+i) + nn of its row
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (!valid[b]) continue;
    const float inv = p.v_scale / acc_l[b][0];
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
