// Paged decode attention on gfx950.
//
// What is computed (bogosort page "五十三：vLLM-PagedAttention" §8, ybb.press
// page "vLLM 与 LLM 推理部署实战" §2.3): for each sequence and query head, the
// query attends every cached token of the sequence, whose K/V are found
// block by block through the block table.
//
// Scheduling.  The grid is persistent: one workgroup per CU, holding as many
// wave64s as the CU keeps resident at the kernel's register count.  Every
// workgroup first reads the batch's lengths into LDS and forms the prefix sum
// of each sequence's count of 32-token steps ("units").  The units of all
// (sequence, KV head) pairs, laid end to end, are cut into equal chunks (about
// one per wave), so every wave streams about the same number of KV bytes
// whatever the length mix.  A chunk that covers a pair partly yields a
// partial result (o, m, l); a pair inside one chunk gets its output written
// directly.  Partials of a pair whose chunks all belong to one workgroup are
// kept in LDS and merged (log-sum-exp) by the last of its waves to finish;
// the others go to the workspace and the reduce kernel merges them.  Two other
// cuts exist: fixed partitions of a given length from each sequence's start,
// and whole pairs (no partials at all).  Each workgroup owns an even share of
// the chunks, or, for the other two cuts, a run of whole items holding about
// an equal share of the units; its waves take them from an LDS queue.
//
// Within a segment a wave walks 32-token steps; K/V are read with 16-byte
// non-temporal loads (each byte is used once).  Block-table entries are read
// with scalar loads one step ahead, so tile addresses are scalar and the
// table reads do not wait on the K/V loads in flight.
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
//
// Cache formats: 16-bit (the query's type), fp8 E4M3 (codes decoded exactly
// with gfx950's packed scaled converts, per-tensor scales folded into the
// logit scale and the output), fp8 K beside a 16-bit V, and int8 with one
// scale per (block, KV head) (codes converted exactly; the block's K scale
// joins each score's scale, its V scale each probability of the value
// product).  For 16-bit caches the newest token of each sequence can be
// taken from the input and written to its slot by the wave that covers it
// (the scatter folded into the decode).
#pragma once

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

constexpr int kStep = 32;       // tokens per step (one unit of work)
constexpr int kMaxPlanSeqs = 8000;
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr int kChunksPerWave = 1;       // balanced cut: chunks per wave, on average

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Issue priority from a wave's progress through its work unit (done of
// total steps, both wave-uniform): the more of it is left, the higher the
// priority, so that waves which lose issue arbitration (the younger ones of
// a SIMD) catch up and the waves of a CU finish together.
__device__ __forceinline__ void progress_priority(int done, int total) {
  const int q = (4 * done) / max(total, 1);
  if (q <= 0) __builtin_amdgcn_s_setprio(3);
  else if (q == 1) __builtin_amdgcn_s_setprio(2);
  else if (q == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Block-table rows are read through the constant address space: uniform
// indices then become scalar loads (the kernels never write the tables).
typedef const __attribute__((address_space(4))) int* ctab_ptr;
typedef const __attribute__((address_space(4))) float* cscale_ptr;   // per-block scales, read-only

// ---------------------------------------------------------------------------
// Plan: clamped lengths and the exclusive prefix sum of per-sequence counts
// (units for the balanced cut, items for the fixed / whole cuts) in LDS.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int plan_count(const DecodeParams& p, int len) {
  const int u = (len + kStep - 1) / kStep;
  if (p.mode == kSplitBalanced) return u;
  if (p.mode == kSplitNone) return u > 0 ? 1 : 0;
  return (u + p.chunk - 1) / p.chunk;
}

template <int NW>
__device__ void build_plan(const DecodeParams& p, int* lens, int* pre) {
  constexpr int NT = 64 * NW;
  __shared__ int wave_sum[NW];
  const int S = p.num_seqs;
  const int per = (S + NT - 1) / NT;
  const int b = min(S, (int)threadIdx.x * per), e = min(S, b + per);
  int sum = 0;
  for (int s = b; s < e; ++s) {
    int n = p.seq_lens[s];
    n = n < 0 ? 0 : (n > p.max_len ? p.max_len : n);
    lens[s] = n;
    const int c = plan_count(p, n);
    pre[s] = c;
    sum += c;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w = 0; w < wave; ++w) run += wave_sum[w];
  for (int s = b; s < e; ++s) {
    const int c = pre[s];
    pre[s] = run;
    run += c;
  }
  if (threadIdx.x == NT - 1) pre[S] = run;
  __syncthreads();
}

// Workgroup share of the fixed and whole cuts' item list: whole items, the
// bounds at the item starts nearest to equal fractions of the batch's
// 32-token units.  Items differ in length (a pair's last partition is
// short), so equal item counts leave the shares' bytes up to ~20 % apart.
// Bound i of workgroup b is the same function of (b + i) in every
// workgroup, so neighbouring shares meet exactly.
template <int NW>
__device__ void unit_share(const DecodeParams& p, const int* lens, const int* pre, int wg, int nwg, int* k0,
                           int* k1) {
  constexpr int NT = 64 * NW;
  __shared__ int wave_units[NW];
  __shared__ int bounds[2];
  const int S = p.num_seqs, H = p.num_kv_heads;
  const int per = (S + NT - 1) / NT;
  const int b = min(S, (int)threadIdx.x * per), e = min(S, b + per);
  int sum = 0;
  for (int s = b; s < e; ++s) sum += (lens[s] + kStep - 1) / kStep;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_units[wave] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) run += wave_units[w];
    total += wave_units[w];
  }
  const int64_t tot = (int64_t)total * H;
  const int64_t x[2] = {tot * wg / nwg, tot * (wg + 1) / nwg};
  int64_t o = (int64_t)run * H;
  for (int s = b; s < e; ++s) {
    const int U = (lens[s] + kStep - 1) / kStep;
    const int64_t end = o + (int64_t)U * H;
    for (int i = 0; i < 2; ++i) {
      if (x[i] >= o && x[i] < end) {
        const int64_t rem = x[i] - o;
        const int h = (int)(rem / U), r = (int)(rem - (int64_t)h * U);
        const int c = p.mode == kSplitNone ? U : p.chunk;   // units per item of this pair
        const int q = pre[s + 1] - pre[s];
        bounds[i] = pre[s] * H + h * q + min(q, (r + c / 2) / c);
      }
    }
    o = end;
  }
  if (threadIdx.x == 0)
    for (int i = 0; i < 2; ++i)
      if (x[i] >= tot) bounds[i] = pre[S] * H;
  __syncthreads();
  *k0 = uni(bounds[0]);
  *k1 = uni(bounds[1]);
}

// Largest s in [0, S) with pre[s] <= x, for 0 <= x < pre[S].
__device__ __forceinline__ int find_seq(const int* pre, int S, int x) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(pre[mid]) <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Partials merged on the CU.  When every partial of a (sequence, KV head)
// pair comes from the same workgroup's share of the work list, the waves put
// them in LDS instead of the workspace, and the last of them to finish
// merges them (log-sum-exp) and stores the output: partial outputs never
// travel to HBM and back.  Pairs that cross a share boundary use the
// workspace and the reduce kernel.
//   slots: [local_slots][group * D] floats, ml: [local_slots][32] (running
//   max of 16 heads, then their sums), cnt: [local_slots] arrival counters.
// Partial `part` of the pair sits in slot stride * (base + part) (+ odd0 for
// part 0); `counter` < 0 marks a pair merged through the workspace.
struct LocalMerge {
  float* slots;
  float* ml;
  int* cnt;
  int base, stride, odd0, counter;
  int prog0, prog_len;   // steps of the wave's work unit done before this segment, and in all
  __device__ __forceinline__ int slot(int part) const { return stride * (base + part) + (part == 0 ? odd0 : 0); }
};

// Block-table entries of one sequence, 128 consecutive ones held as two
// registers per lane; entry b is read out with v_readlane.
template <int BS>
struct TableWindow {
  const int* row;
  int nblk;
  int base;   // multiple of 64
  int a, b;   // entries base + lane, base + 64 + lane

  __device__ __forceinline__ void init(const int* r, int n, int first) {
    const int lane = threadIdx.x & 63;
    row = r;
    nblk = n;
    base = first & ~63;
    a = (base + lane < nblk) ? row[base + lane] : 0;
    b = (base + 64 + lane < nblk) ? row[base + 64 + lane] : 0;
  }
  // Make entries up to `last` readable.  Callers advance by at most two
  // blocks at a time, and a step's blocks never straddle a multiple of 64.
  __device__ __forceinline__ void ensure(int last) {
    if (last >= base + 64) {
      const int lane = threadIdx.x & 63;
      base += 64;
      a = b;
      b = (base + 64 + lane < nblk) ? row[base + 64 + lane] : 0;
    }
  }
  __device__ __forceinline__ int get(int bi) const {
    const int r = bi - base;
    return r < 64 ? __builtin_amdgcn_readlane(a, r) : __builtin_amdgcn_readlane(b, r - 64);
  }
};

// ---------------------------------------------------------------------------
// MFMA segment for 16-bit, fp8 and int8 caches.
//   QT: query / output / MFMA operand type (__bf16 or _Float16)
//   KF, VF: element format of the K / V pool: kFmtQ (QT itself), kFmtFp8
//   (E4M3 codes, decoded exactly to QT) or kFmtI8 (int8 codes with one
//   float32 scale per (block, KV head), in p.k_scales / p.v_scales).  K fp8
//   with V in QT is the mixed format of the intelliparadigm page §6.1 (fp8 K
//   cache, bf16 V cache).
// ---------------------------------------------------------------------------
enum : int { kFmtQ = 0, kFmtFp8 = 1, kFmtI8 = 2 };

// APPEND: the newest token of every sequence (position seq_len - 1) comes
// from p.new_k / p.new_v: the wave whose segment covers it first stores its
// K and V rows into the pool slot, then reads the whole context from the
// pool (the scatter folded into the decode; 16-bit caches only).
template <typename QT, int KF, int VF, int D, int BS, bool APPEND = false>
struct MfmaDecode {
  static constexpr bool KF8 = KF != kFmtQ, VF8 = VF != kFmtQ;   // one byte per element
  static constexpr bool kBlockScales = KF == kFmtI8;             // K and V int8 together
  // Rescaling slack (log2 units).  With int8 blocks the value operand is
  // p * (block V scale) in QT; f16's range (65504) then needs p <= 1, i.e.
  // the reference max always equal to the running max.
  static constexpr float kSlack = (kBlockScales && __is_same(QT, _Float16)) ? 0.0f : kRescaleSlack;
  static constexpr int NC = D / 32;             // QK MFMAs per 16-token tile
  static constexpr int DPL = D / 16;            // value dims per lane = PV MFMAs per step
  static constexpr int KEB = KF8 ? 1 : 2, VEB = VF8 ? 1 : 2;
  static constexpr int VW = DPL * VEB / 4;      // dwords per V row piece
  static constexpr int KL = KF8 ? D / 64 : NC;  // 16-byte K loads per lane and tile
  static constexpr bool kDoubleBuffer = KF8 && VF8;
  // 8-bit K rows (128 B at D = 128) are read a whole cache line per 8 lanes
  // and put into the matrix-core layout (one row per lane) through 4 KB of
  // the wave's LDS: whole-line requests carry twice the bytes of the
  // half-line pieces the layout asks for (measured faster with 8-bit V,
  // slower beside a 16-bit V)
  static constexpr bool kStageK = KF8 && VF8 && D == 128 && BS >= 16 && !APPEND;
  // partials of pairs inside one workgroup's share are merged in LDS
  static constexpr bool kLocalMerge = true;
  // waves per workgroup = waves one CU keeps resident at this register count
  // (int8 at D = 64 needs a few registers more than 16 waves allow)
  static constexpr int kWaves = D == 64 ? (kBlockScales ? 12 : 16) : (KF8 && VF8 ? 8 : 12);

  struct Buf {
    u32x4 k[2][KL];
    uint32_t v[2][4][VW];
    float ks[2], vs[2];   // int8: scales of the blocks of this lane's score rows (per tile)
  };

  // Block ids of step j, read with scalar loads (constant address space:
  // they are counted apart from the vector loads in flight): b[tau] holds
  // the block of 16-token tile tau, or, for 8-token blocks, b[2 tau + half]
  // that of each half tile.  A block past the end is replaced by the last one
  // (its tokens are masked).
  static constexpr int NID = BS < 16 ? 4 : 2;
  struct Ids {
    int b[NID];
  };
  static __device__ __forceinline__ Ids ids(ctab_ptr row, int nblk, int j) {
    Ids r;
#pragma unroll
    for (int q = 0; q < NID; ++q) r.b[q] = row[min((j * kStep + (kStep / NID) * q) / BS, nblk - 1)];
    return r;
  }

  // Issue the loads of step j (tokens 32j .. 32j+31 of the pair).
  static __device__ __forceinline__ void load(Buf& buf, Ids id, const DecodeParams& p, int kvh, int j) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, c16 = lane & 15;
    const char* kpool = reinterpret_cast<const char*>(p.k_pool);
    const char* vpool = reinterpret_cast<const char*>(p.v_pool);
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      // element offsets of this lane's K row and of its first V row
      int64_t krow, vrow;
      if constexpr (BS < 16) {
        // 8-token blocks: rows 0-7 and 8-15 of the tile lie in two blocks
        const int kb = c16 < 8 ? id.b[2 * tau] : id.b[2 * tau + 1];
        const int vb = G < 2 ? id.b[2 * tau] : id.b[2 * tau + 1];
        krow = (((int64_t)kb * p.num_kv_heads + kvh) * BS + (c16 & 7)) * D;
        vrow = (((int64_t)vb * p.num_kv_heads + kvh) * BS + 4 * (G & 1)) * D;
      } else {
        const int row0 = (j * kStep + 16 * tau) % BS;
        const int64_t tile = (((int64_t)id.b[tau] * p.num_kv_heads + kvh) * BS + row0) * D;  // elements
        krow = tile + (int64_t)c16 * D;
        vrow = tile + (int64_t)(4 * G) * D;
      }
      if constexpr (kBlockScales) {
        // the lane's score rows (tokens 4 G .. 4 G + 3 of the tile) lie in
        // block id.b[tau], or, for 8-token blocks, in half G / 2 of the tile
        const int b0 = BS < 16 ? id.b[2 * tau] : id.b[tau];
        const int b1 = BS < 16 ? id.b[2 * tau + 1] : id.b[tau];
        const cscale_ptr ksp = (cscale_ptr)p.k_scales, vsp = (cscale_ptr)p.v_scales;
        const int64_t i0 = (int64_t)b0 * p.num_kv_heads + kvh, i1 = (int64_t)b1 * p.num_kv_heads + kvh;
        const float k0 = ksp[i0], k1 = ksp[i1], v0 = vsp[i0], v1 = vsp[i1];
        buf.ks[tau] = G < 2 ? k0 : k1;
        buf.vs[tau] = G < 2 ? v0 : v1;
      }
      const char* kt = kpool + krow * KEB;
      if constexpr (kStageK) {
        // instruction h: rows 8 h + 2 G + c16 / 8 of the tile, 16 bytes each
        const char* kr = kt - (int64_t)c16 * D;   // row 0 of the tile
#pragma unroll
        for (int h = 0; h < KL; ++h) buf.k[tau][h] = ld16_nt(kr + (8 * h + 2 * G + (c16 >> 3)) * D + 16 * (c16 & 7));
      } else if constexpr (KF8) {
#pragma unroll
        for (int h = 0; h < KL; ++h) buf.k[tau][h] = ld16_nt(kt + 64 * h + 16 * G);
      } else {
#pragma unroll
        for (int c = 0; c < KL; ++c) buf.k[tau][c] = ld16_nt(kt + (32 * c + 8 * G) * 2);
      }
      const char* vt = vpool + (vrow + DPL * c16) * VEB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* src = vt + (int64_t)i * D * VEB;
        if constexpr (VW == 4) {
          const u32x4 x = ld16_nt(src);
          buf.v[tau][i][0] = x.x; buf.v[tau][i][1] = x.y; buf.v[tau][i][2] = x.z; buf.v[tau][i][3] = x.w;
        } else if constexpr (VW == 2) {
          const u32x2 x = ld8_nt(src);
          buf.v[tau][i][0] = x.x; buf.v[tau][i][1] = x.y;
        } else {
          buf.v[tau][i][0] = ld4_nt(src);
        }
      }
    }
  }

  // m: the reference max (log2 units); l4: the sums of the rounded
  // probabilities, formed on the matrix cores by a value product against an
  // all-ones operand (every element of a lane's l4 holds its head's sum over
  // all the tokens so far), or for an int8 cache the float32 probabilities
  // summed per lane in l4[0] (the head's four lanes are added at the end);
  // acc: the unnormalised output.
  struct State {
    float m;
    f32x4 l4;
    f32x4 acc[DPL];
  };

  struct NoHook {
    __device__ __forceinline__ void operator()() const {}
  };

  // One step's products and softmax.  `after_scores` runs once the step's
  // score products are issued, i.e. after the 8-bit K staging's LDS reads
  // were waited for: scalar loads issued there (block ids of a later step)
  // are not covered by that wait.
  template <class Hook = NoHook>
  static __device__ __forceinline__ void compute(Buf& buf, State& st, const u32x4 (&qop)[NC],
                                                 float qk_scale_log2, int len, int j,
                                                 char* kst = nullptr, Hook after_scores = Hook()) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4;
    const int rel0 = j * kStep;
    // rows past the end hold stale or poisoned data: zero their values
    // (a zero probability does not cancel a NaN in the product)
    if (rel0 + kStep > len) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rel0 + 16 * tau + 4 * G + i >= len) {
#pragma unroll
            for (int w = 0; w < VW; ++w) buf.v[tau][i][w] = 0u;
          }
    }
    // Scores: S^T tile tau, lane (G, c16) holds tokens 4G+i of head c16.
    float s[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      u32x4 ka[NC];
      if constexpr (kStageK) {
        // whole-line rows to the layout of the score product: row c16, the
        // 16-byte pieces 4 h + G (pieces XOR-swizzled by row in LDS)
        const int c16 = lane & 15;
        char* sb = kst + tau * 2048;
        // the buffer is the wave's own: the last step's reads of it (by
        // other lanes of this wave) come before it is overwritten
        if (tau == 0) wave_lds_acquire();
#pragma unroll
        for (int h = 0; h < KL; ++h) {
          const int r = 8 * h + 2 * G + (c16 >> 3);
          *reinterpret_cast<u32x4*>(sb + r * 128 + (((c16 & 7) ^ (r & 7)) * 16)) = buf.k[tau][h];
        }
        // each lane reads pieces other lanes of the wave stored just above
        wave_lds_release();
        wave_lds_acquire();
#pragma unroll
        for (int h = 0; h < KL; ++h)
          buf.k[tau][h] = *reinterpret_cast<const u32x4*>(sb + c16 * 128 + (((4 * h + G) ^ (c16 & 7)) * 16));
        if (tau == 1) wave_lds_release();
      }
      if constexpr (KF == kFmtFp8) {
#pragma unroll
        for (int h = 0; h < KL; ++h) {
          const u32x4 raw = buf.k[tau][h];
          ka[2 * h] = u32x4{fp8x2_to<QT>(raw.x, false), fp8x2_to<QT>(raw.x, true),
                            fp8x2_to<QT>(raw.y, false), fp8x2_to<QT>(raw.y, true)};
          ka[2 * h + 1] = u32x4{fp8x2_to<QT>(raw.z, false), fp8x2_to<QT>(raw.z, true),
                                fp8x2_to<QT>(raw.w, false), fp8x2_to<QT>(raw.w, true)};
        }
      } else if constexpr (KF == kFmtI8) {
#pragma unroll
        for (int h = 0; h < KL; ++h) {
          const u32x4 raw = buf.k[tau][h];
          ka[2 * h] = u32x4{i8x2_to<QT>(raw.x, false), i8x2_to<QT>(raw.x, true),
                            i8x2_to<QT>(raw.y, false), i8x2_to<QT>(raw.y, true)};
          ka[2 * h + 1] = u32x4{i8x2_to<QT>(raw.z, false), i8x2_to<QT>(raw.z, true),
                                i8x2_to<QT>(raw.w, false), i8x2_to<QT>(raw.w, true)};
        }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[c] = buf.k[tau][c];
      }
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sc = Mma<QT>::mma(ka[c], qop[c], sc);
      if (tau == 1) after_scores();
      // int8: the block's K scale joins the logit scale
      const float cs = kBlockScales ? qk_scale_log2 * buf.ks[tau] : qk_scale_log2;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[tau][i] = mul_rn(sc[i], cs);
    }
    // tokens past the end (only in a pair's last step) take logit -inf
    if (rel0 + kStep > len) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rel0 + 16 * tau + 4 * G + i >= len) s[tau][i] = -INFINITY;
    }
    float smax = fmax_nan(fmax_nan(fmax_nan(s[0][0], s[0][1]), fmax_nan(s[0][2], s[0][3])),
                          fmax_nan(fmax_nan(s[1][0], s[1][1]), fmax_nan(s[1][2], s[1][3])));
    smax = lanes4_max(smax);
    // Lazy rescaling: the reference max moves (and the accumulators are
    // rescaled) only when some head's max exceeds it by more than the slack,
    // so probabilities stay <= 2^slack.  The first step always sets it (st.m
    // starts at -inf; every step has a valid token).
    if (__builtin_amdgcn_ballot_w64(smax > st.m + kSlack) != 0) {
      const float m_new = fmaxf(st.m, smax);
      const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
      st.m = m_new;
      st.l4 = st.l4 * alpha;
#pragma unroll
      for (int n = 0; n < DPL; ++n) st.acc[n] = st.acc[n] * alpha;
    }
    uint32_t pw[4];
    float ls = 0.f;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float a = __builtin_amdgcn_exp2f(s[tau][i] - st.m);
        const float b = __builtin_amdgcn_exp2f(s[tau][i + 1] - st.m);
        // int8: the value operand carries the block's V scale, rounded once
        // with the probability; the sum takes the float32 probabilities, so
        // each weight of the normalised output carries a single rounding
        if constexpr (kBlockScales) {
          pw[tau * 2 + i / 2] = pack2<QT>(a * buf.vs[tau], b * buf.vs[tau]);
          ls += a + b;
        } else {
          pw[tau * 2 + i / 2] = pack2<QT>(a, b);
        }
      }
    }
    const u32x4 pop = {pw[0], pw[1], pw[2], pw[3]};
    // 16-bit and fp8: the sum of the rounded probabilities (so that the
    // weights stay normalised), their product with an all-ones operand
    if constexpr (kBlockScales)
      st.l4[0] += ls;
    else
      st.l4 = Mma<QT>::mma(u32x4{kOnes<QT>, kOnes<QT>, kOnes<QT>, kOnes<QT>}, pop, st.l4);

    // Values: A operand for dim DPL*c16 + n holds tokens 4G+0..3 of tile 0
    // then 4G+0..3 of tile 1.
#pragma unroll
    for (int n = 0; n < DPL; ++n) {
      u32x4 a;
      if constexpr (VF8) {
        const int w = n >> 2, k = n & 3;
        uint32_t x[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const uint32_t r0 = buf.v[tau][0][w], r1 = buf.v[tau][1][w];
          const uint32_t r2 = buf.v[tau][2][w], r3 = buf.v[tau][3][w];
          const uint32_t ta = (k & 1) ? perm(r1, r0, 0x07030501u) : perm(r1, r0, 0x06020400u);
          const uint32_t tc = (k & 1) ? perm(r3, r2, 0x07030501u) : perm(r3, r2, 0x06020400u);
          x[tau] = (k & 2) ? perm(tc, ta, 0x07060302u) : perm(tc, ta, 0x05040100u);
        }
        if constexpr (VF == kFmtI8)
          a = u32x4{i8x2_to<QT>(x[0], false), i8x2_to<QT>(x[0], true),
                    i8x2_to<QT>(x[1], false), i8x2_to<QT>(x[1], true)};
        else
          a = u32x4{fp8x2_to<QT>(x[0], false), fp8x2_to<QT>(x[0], true),
                    fp8x2_to<QT>(x[1], false), fp8x2_to<QT>(x[1], true)};
      } else {
        const int w = n >> 1;
        const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
        a = u32x4{perm(buf.v[0][1][w], buf.v[0][0][w], sel), perm(buf.v[0][3][w], buf.v[0][2][w], sel),
                  perm(buf.v[1][1][w], buf.v[1][0][w], sel), perm(buf.v[1][3][w], buf.v[1][2][w], sel)};
      }
      st.acc[n] = Mma<QT>::mma(a, pop, st.acc[n]);
    }
  }

  // Output rows of query head hq: v_scale * acc / l_tot in QT (lanes of the
  // head's column).
  static __device__ __forceinline__ void store_output(const DecodeParams& p, const f32x4 (&acc)[DPL],
                                                      float l_tot, int s, int hq) {
    const int G = (threadIdx.x & 63) >> 4;
    QT* orow = reinterpret_cast<QT*>(p.out) + ((int64_t)s * p.num_q_heads + hq) * D;
    const float inv = p.v_scale / l_tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[DPL / 2];
#pragma unroll
      for (int n = 0; n < DPL; n += 2) w[n / 2] = pack2<QT>(acc[n][i] * inv, acc[n + 1][i] * inv);
      QT* dst = orow + DPL * (4 * G + i);
      if constexpr (DPL == 8) st16(dst, u32x4{w[0], w[1], w[2], w[3]});
      else *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
    }
  }

  // This wave's partial goes to its LDS slot; the last of the pair's waves
  // to arrive merges all of them and stores the output.  A lane keeps the
  // same (head, dims) in every slot, so the merge is lane-local.
  static __device__ __forceinline__ void merge_local(const DecodeParams& p, f32x4 (&acc)[DPL], float m,
                                                     float l_tot, int s, int kvh, int part, int nparts,
                                                     const LocalMerge& lm) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, c16 = lane & 15;
    const int g = p.group;
    if (part == 0 && p.nparts != nullptr && lane == 0) p.nparts[s * p.num_kv_heads + kvh] = 1;  // merged here
    const int lq = G * g + c16;   // this lane's position among the 4 g writing lanes
    if (c16 < g) {
      float* dst = lm.slots + (int64_t)lm.slot(part) * g * D;
#pragma unroll
      for (int k = 0; k < DPL; ++k)   // quad k = (i, nq): acc[4 nq + e][i]
        *reinterpret_cast<f32x4*>(dst + (k * 4 * g + lq) * 4) =
            f32x4{acc[4 * (k % (DPL / 4))][k / (DPL / 4)], acc[4 * (k % (DPL / 4)) + 1][k / (DPL / 4)],
                  acc[4 * (k % (DPL / 4)) + 2][k / (DPL / 4)], acc[4 * (k % (DPL / 4)) + 3][k / (DPL / 4)]};
      if (G == 0) {
        lm.ml[lm.slot(part) * 32 + c16] = m;
        lm.ml[lm.slot(part) * 32 + 16 + c16] = l_tot;
      }
    }
    __threadfence_block();
    int old = 0;
    if (lane == 0) old = atomicAdd(&lm.cnt[lm.counter], 1);
    old = __builtin_amdgcn_readlane(old, 0);
    if (old != nparts - 1) return;
    __threadfence_block();
    if (c16 >= g) return;
    float M = -INFINITY;
    for (int t = 0; t < nparts; ++t) M = fmaxf(M, lm.ml[lm.slot(t) * 32 + c16]);
    // acc (this wave's own partial, already in its slot) becomes the sum
#pragma unroll
    for (int n = 0; n < DPL; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int t = 0; t < nparts; ++t) {
      const int sl = lm.slot(t);
      const float w = __builtin_amdgcn_exp2f(lm.ml[sl * 32 + c16] - M);
      L += w * lm.ml[sl * 32 + 16 + c16];
      const float* src = lm.slots + (int64_t)sl * g * D;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + (k * 4 * g + lq) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * (k % (DPL / 4)) + e][k / (DPL / 4)] += w * x[e];
      }
    }
    store_output(p, acc, L, s, kvh * g + c16);
  }

  // One wave: steps [j0, j1) of pair (s, kvh), then the output or a partial.
  static __device__ void segment(const DecodeParams& p, int s, int kvh, int len, int j0, int j1,
                                 int part, int nparts, const LocalMerge& lm) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, c16 = lane & 15;
    const int g = p.group;

    // Query operand (B of S^T = K Q^T): head column c16, 8 dims per MFMA.
    // The dims a lane group covers in MFMA c follow the order in which K row
    // pieces are loaded (any permutation of the reduction index is allowed as
    // long as K and Q agree).
    u32x4 qop[NC];
    {
      const QT* qrow = reinterpret_cast<const QT*>(p.q) +
                       ((int64_t)s * p.num_q_heads + kvh * g + c16) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int d0 = KF8 ? (64 * (c >> 1) + 16 * G + 8 * (c & 1)) : (32 * c + 8 * G);
        qop[c] = (c16 < g) ? ld16(qrow + d0) : u32x4{0, 0, 0, 0};
      }
    }

    const ctab_ptr trow = (ctab_ptr)(p.block_tables + (int64_t)s * p.max_blocks);
    const int nblk = (len + BS - 1) / BS;
    // APPEND: the segment that covers the newest token loads its K and V rows
    // (lanes 0-31: K, 32-63: V; D / 16 bytes each) here and stores them in
    // the pool slot once its first step's loads are on their way (before
    // them if that step is the last one); the last step reads them back from
    // the pool
    const bool appends = APPEND && len > 0 && j1 == (len + kStep - 1) / kStep;
    u32x2 new_row = {0u, 0u};
    char* new_dst = nullptr;
    if constexpr (APPEND) {
      if (appends) {
        const bool is_v = lane >= 32;
        const char* src = reinterpret_cast<const char*>(is_v ? p.new_v : p.new_k) +
                          ((int64_t)s * (is_v ? p.new_v_stride : p.new_k_stride) + (int64_t)kvh * D) * 2;
        const int b = (lane & 31) * (D / 16);
        if constexpr (D == 128) new_row = *reinterpret_cast<const u32x2*>(src + b);
        else new_row.x = *reinterpret_cast<const uint32_t*>(src + b);
        const int pos = len - 1;
        const int64_t off = (((int64_t)trow[pos / BS] * p.num_kv_heads + kvh) * BS + pos % BS) * D * 2;
        new_dst = reinterpret_cast<char*>(const_cast<void*>(is_v ? p.v_pool : p.k_pool)) + off + b;
      }
    }
    auto store_new_row = [&]() {
      if constexpr (D == 128) *reinterpret_cast<u32x2*>(new_dst) = new_row;
      else *reinterpret_cast<uint32_t*>(new_dst) = new_row.x;
    };
    extern __shared__ __align__(16) int plan_lds[];
    char* kst = kStageK ? reinterpret_cast<char*>(plan_lds) + p.kstage_off + (threadIdx.x >> 6) * 4096 : nullptr;

    State st;
    st.m = -INFINITY;
    st.l4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < DPL; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The block ids of the next step are fetched one step ahead.  With
    // kDoubleBuffer the K/V loads of step j+1 are in flight while step j is
    // computed (two register buffers); otherwise one buffer keeps the
    // register count low enough for more waves per SIMD.
    Ids cur = ids(trow, nblk, j0);
    if constexpr (kDoubleBuffer) {
      // Block ids are fetched two steps ahead: those of step j + 3 while step
      // j is computed, after its K staging (see compute), so that neither an
      // LDS wait nor the next step's loads wait for them.
      Buf A, B;
      Ids n1 = ids(trow, nblk, min(j0 + 1, j1 - 1));
      Ids n2 = ids(trow, nblk, min(j0 + 2, j1 - 1));
      load(A, cur, p, kvh, j0);
      for (int j = j0; j < j1; j += 2) {
        if (lm.prog_len > 0) progress_priority(lm.prog0 + j - j0, lm.prog_len);
        Ids n3, n4;
        if (j + 1 < j1) load(B, n1, p, kvh, j + 1);
        compute(A, st, qop, p.qk_scale_log2, len, j, kst,
                [&] { n3 = ids(trow, nblk, min(j + 3, j1 - 1)); });
        if (j + 1 >= j1) break;
        if (j + 2 < j1) load(A, n2, p, kvh, j + 2);
        compute(B, st, qop, p.qk_scale_log2, len, j + 1, kst,
                [&] { n4 = ids(trow, nblk, min(j + 4, j1 - 1)); });
        n1 = n3;
        n2 = n4;
      }
    } else {
      int jfirst = j0;
      if constexpr (APPEND) {
        // the first step of an appending segment, peeled so that the new
        // rows' registers are free in the loop
        if (appends) {
          const Ids nxt = ids(trow, nblk, min(j0 + 1, j1 - 1));
          if (j0 == j1 - 1) {
            store_new_row();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
          }
          Buf buf;
          load(buf, cur, p, kvh, j0);
          if (j0 < j1 - 1) store_new_row();
          compute(buf, st, qop, p.qk_scale_log2, len, j0, kst);
          cur = nxt;
          jfirst = j0 + 1;
        }
      }
      for (int j = jfirst; j < j1; ++j) {
        if (lm.prog_len > 0) progress_priority(lm.prog0 + j - j0, lm.prog_len);
        const Ids nxt = ids(trow, nblk, min(j + 1, j1 - 1));
        if constexpr (APPEND) {
          if (appends && j == j1 - 1) {
            // other lanes of this wave read the rows stored in the first
            // step in this step's loads
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
          }
        }
        Buf buf;
        load(buf, cur, p, kvh, j);
        compute(buf, st, qop, p.qk_scale_log2, len, j, kst);
        cur = nxt;
      }
    }
    // lane (G, c16) holds head c16, dims DPL*(4G+i) + n
    const float l_tot = kBlockScales ? lanes4_sum(st.l4[0]) : st.l4[0];
    if constexpr (kLocalMerge) {
      if (nparts > 1 && lm.counter >= 0) {
        merge_local(p, st.acc, st.m, l_tot, s, kvh, part, nparts, lm);
        return;
      }
    }
    if (c16 < g) {
      const int hq = kvh * g + c16;
      if (nparts == 1) {
        store_output(p, st.acc, l_tot, s, hq);
      } else {
        const int64_t b = ((int64_t)s * p.num_q_heads + hq) * p.max_parts + part;
        float* o = p.part_o + b * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* dst = o + DPL * (4 * G + i);
#pragma unroll
          for (int n = 0; n < DPL; n += 4)
            *reinterpret_cast<f32x4*>(dst + n) =
                f32x4{st.acc[n][i], st.acc[n + 1][i], st.acc[n + 2][i], st.acc[n + 3][i]};
        }
        if (G == 0) {
          p.part_m[b] = st.m;
          p.part_l[b] = l_tot;
        }
      }
    }
    if (part == 0 && p.nparts != nullptr && lane == 0) p.nparts[s * p.num_kv_heads + kvh] = nparts;
  }
};

// ---------------------------------------------------------------------------
// fp32 segment (VALU): the small fp32 workloads.  The head dimension is
// spread over the lanes; tokens are taken one at a time from groups of 16
// whose rows were loaded together.
// ---------------------------------------------------------------------------
template <int D, int BS>
struct F32Decode {
  static constexpr int kWaves = D == 64 ? 12 : 8;  // resident waves per CU
  static constexpr bool kLocalMerge = false;
  static constexpr bool kStageK = false;
  static __device__ void segment(const DecodeParams& p, int s, int kvh, int len, int j0, int j1,
                                 int part, int nparts, const LocalMerge&) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int g = p.group;
    const float* q = reinterpret_cast<const float*>(p.q) + ((int64_t)s * p.num_q_heads + kvh * g) * D;
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
    TableWindow<BS> win;
    win.init(p.block_tables + (int64_t)s * p.max_blocks, (len + BS - 1) / BS, (j0 * kStep) / BS);
    const float* kpool = reinterpret_cast<const float*>(p.k_pool);
    const float* vpool = reinterpret_cast<const float*>(p.v_pool);
    const int t_end = min(j1 * kStep, len);
    // 16 tokens' rows are loaded before any is used, so one memory latency
    // covers 16 tokens (past the end, the last token's row is re-read).
    constexpr int kGroup = 16;
    for (int t0 = j0 * kStep; t0 < t_end; t0 += kGroup) {
      float kv[kGroup][E], vv[kGroup][E];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        const int t = min(t0 + k, t_end - 1);
        const int bi = t / BS;
        win.ensure(bi);
        const int blk = win.get(bi);
        const int64_t rowoff = (((int64_t)blk * p.num_kv_heads + kvh) * BS + t % BS) * D;
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
            for (int msk = 32; msk >= 1; msk >>= 1) dot = xor_sum(dot, msk);
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
        const int hq = kvh * g + j;
        if (nparts == 1) {
          float* orow = reinterpret_cast<float*>(p.out) + ((int64_t)s * p.num_q_heads + hq) * D;
          const float inv = p.v_scale / l[j];
#pragma unroll
          for (int e = 0; e < E; ++e) orow[lane + 64 * e] = acc[j][e] * inv;
        } else {
          const int64_t b = ((int64_t)s * p.num_q_heads + hq) * p.max_parts + part;
#pragma unroll
          for (int e = 0; e < E; ++e) p.part_o[b * D + lane + 64 * e] = acc[j][e];
          if (lane == 0) {
            p.part_m[b] = m[j];
            p.part_l[b] = l[j];
          }
        }
      }
    }
    if (part == 0 && p.nparts != nullptr && lane == 0) p.nparts[s * p.num_kv_heads + kvh] = nparts;
  }
};

// ---------------------------------------------------------------------------
// Work of the balanced cut: chunk k covers units [k*chunk, (k+1)*chunk) of
// the unit line, i.e. one or more segments.  Chunk boundaries are fixed by
// the chunk size alone, so the partial index of a segment (its chunk minus
// the first chunk of its pair) does not depend on which wave runs it.
// ---------------------------------------------------------------------------
template <class Seg>
__device__ __forceinline__ void run_chunk(const DecodeParams& p, const int* lens, const int* pre,
                                          int T, int chunk, int k, LocalMerge lm, int k0, int k1) {
  const int S = p.num_seqs, H = p.num_kv_heads;
  const int ustart = k * chunk;
  int u = ustart;
  const int uend = min(T, u + chunk);
  int s = find_seq(pre, S, u / H);
  int base = uni(pre[s]);
  int U = uni(pre[s + 1]) - base;
  int h = (u - base * H) / U;
  int j = u - base * H - h * U;
  while (true) {
    const int ps = base * H + h * U;  // first unit of the pair
    const int j1 = min(U, j + (uend - u));
    const int wf = ps / chunk, wl = (ps + U - 1) / chunk;
    // chunk k' holds its pair partials in slots 2 (k' - k0) (the one that
    // continues a pair) and 2 (k' - k0) + 1 (the one that starts a pair
    // after the chunk's start)
    lm.base = wf - k0;
    lm.odd0 = ps % chunk != 0;
    lm.counter = (lm.slots != nullptr && wf >= k0 && wl < k1) ? wf - k0 : -1;
    lm.prog0 = u - ustart;
    lm.prog_len = uend - ustart;
    Seg::segment(p, s, h, uni(lens[s]), j, j1, k - wf, wl - wf + 1, lm);
    u += j1 - j;
    if (u >= uend) break;
    j = 0;
    if (++h == H) {
      h = 0;
      do {
        ++s;
      } while (uni(pre[s + 1]) == uni(pre[s]));
      base = uni(pre[s]);
      U = uni(pre[s + 1]) - base;
    }
  }
}

// Work item i of the fixed and whole cuts: one partition of one pair.
template <class Seg>
__device__ __forceinline__ void run_item(const DecodeParams& p, const int* lens, const int* pre,
                                         int i, LocalMerge lm, int k0, int k1) {
  const int S = p.num_seqs, H = p.num_kv_heads;
  const int s = find_seq(pre, S, i / H);
  const int base = uni(pre[s]);
  const int q = uni(pre[s + 1]) - base;
  const int rel = i - base * H;
  const int h = rel / q, part = rel - h * q;
  const int len = uni(lens[s]);
  const int U = (len + kStep - 1) / kStep;
  const int j0 = part * p.chunk;
  const int j1 = min(U, j0 + p.chunk);
  // item i' holds its partial in slot i' - k0
  const int first = i - part;
  lm.base = first - k0;
  lm.odd0 = 0;
  lm.counter = (lm.slots != nullptr && first >= k0 && first + q <= k1) ? first - k0 : -1;
  lm.prog0 = 0;
  lm.prog_len = 0;   // items differ in length and come from a queue: no progress priority
  Seg::segment(p, s, h, len, j0, j1, part, q, lm);
}

// Next ticket of the workgroup's queue (LDS counter), the same in all lanes.
__device__ __forceinline__ int take_ticket(int* counter) {
  int v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(counter, 1);
  return __builtin_amdgcn_readlane(v, 0);
}

// ---------------------------------------------------------------------------
// One workgroup's part of a decode call: workgroup wg of nwg (NW waves).
// Plan, zero outputs of empty sequences (every nwg-th sequence from wg),
// then the waves take the workgroup's share of the work list from an LDS
// queue.  `pick` may lower nwg once the plan (the clamped lengths in LDS)
// is known; it must return the same count in every workgroup.  The decode
// kernel runs it as one persistent workgroup per CU holding all the waves
// the CU keeps resident; the mixed-step kernel runs it in workgroups of four
// waves beside prefill tiles.
//
// Finer chunks (several per wave, so that fast waves could take more of
// them) were measured slower on MI355X: each extra chunk adds a segment
// start and a partial, which cost more than the balance gains.  Items of the
// fixed and whole cuts differ in length, and there the queue does balance.
// ---------------------------------------------------------------------------
// Workgroup count of a decode launch: all of them take shares.
struct AllShares {
  __device__ int operator()(const int* /*lens*/, int /*S*/, int nwg) const { return nwg; }
};

template <class Seg, typename QT, int NW, class Pick = AllShares>
__device__ __forceinline__ void decode_share(const DecodeParams& p, int wg, int nwg, const Pick& pick = Pick()) {
  constexpr int NT = 64 * NW;
  extern __shared__ __align__(16) int plan_lds[];
  __shared__ int queue;
  const int S = p.num_seqs, H = p.num_kv_heads;
  int* lens = plan_lds;
  int* pre = plan_lds + S;
  // slots for partials merged on the CU, after the plan (16-byte aligned)
  const int nslots = p.local_slots;
  int* cnt = plan_lds + ((2 * S + 1 + 3) & ~3);
  float* ml = reinterpret_cast<float*>(cnt + ((nslots + 3) & ~3));
  float* slots = ml + 32 * nslots;
  if (threadIdx.x == 0) queue = 0;
  for (int i = threadIdx.x; i < nslots; i += NT) cnt[i] = 0;
  build_plan<NW>(p, lens, pre);  // ends with a barrier
  // how many of the nwg workgroups take shares (the same in all of them);
  // the others have nothing to do
  nwg = pick(lens, S, nwg);
  if (wg >= nwg) return;

  // Sequences with no tokens get a zero output (and a partial count of 0).
  for (int s = wg; s < S; s += nwg) {
    if (lens[s] == 0) {
      QT* out = reinterpret_cast<QT*>(p.out) + (int64_t)s * p.num_q_heads * p.head_dim;
      for (int i = threadIdx.x; i < p.num_q_heads * p.head_dim; i += NT) out[i] = (QT)0.0f;
      if (p.nparts != nullptr)
        for (int h = threadIdx.x; h < H; h += NT) p.nparts[s * H + h] = 0;
    }
  }

  // Work list: chunks of units (balanced cut) or items (fixed / whole cuts).
  const int T = uni(pre[S]) * H;
  int chunk = 1, nwork = T;
  if (p.mode == kSplitBalanced) {
    const int64_t want = (int64_t)nwg * NW * kChunksPerWave;
    chunk = (int)((T + want - 1) / want);
    chunk = chunk < p.chunk ? p.chunk : chunk;
    nwork = (T + chunk - 1) / chunk;
  }
  int k0, k1;
  if (p.mode == kSplitBalanced) {
    k0 = (int)((int64_t)nwork * wg / nwg);
    k1 = (int)((int64_t)nwork * (wg + 1) / nwg);
  } else {
    unit_share<NW>(p, lens, pre, wg, nwg, &k0, &k1);
  }
  // local merging needs a slot for every partial of the share
  LocalMerge lm;
  const int need = p.mode == kSplitBalanced ? 2 * (k1 - k0) : k1 - k0;
  lm.slots = (nslots > 0 && need <= nslots && p.mode != kSplitNone) ? slots : nullptr;
  lm.ml = ml;
  lm.cnt = cnt;
  lm.stride = p.mode == kSplitBalanced ? 2 : 1;
  lm.base = 0;
  lm.odd0 = 0;
  lm.counter = -1;
  lm.prog0 = 0;
  lm.prog_len = 1;
  for (int k = k0 + take_ticket(&queue); k < k1; k = k0 + take_ticket(&queue)) {
    if (p.mode == kSplitBalanced) run_chunk<Seg>(p, lens, pre, T, chunk, k, lm, k0, k1);
    else run_item<Seg>(p, lens, pre, k, lm, k0, k1);
  }
}

}  // namespace pa
