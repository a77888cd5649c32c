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
// 64-key tiles held in two LDS stages: while tile t is computed, tile t + 1
// is copied from HBM straight into the other stage by LDS-DMA loads (no
// registers, no LDS stores); one barrier per tile hands the stages over.
// Each wave (32 query rows) forms
//   S^T[key][row] = K[key][:] . Q[row][:]            (v_mfma_f32_16x16x32)
//   O^T[dim][row] += V^T[dim][key] P^T[key][row]     (v_mfma_f32_16x16x32)
// with an online softmax per query row.  As in the decode kernel, the score
// tile's register layout is the value product's B operand, so
// probabilities stay in their lanes; the value operand V^T is read from the
// row-major V tile with gfx950's transposing LDS reads (ds_read_b64_tr_b16).
//
// An fp8 E4M3 cache (ybb.press page §6.2, KV cache in FP8) is staged through
// registers instead: the next tile's codes are loaded while the current one
// is computed, then decoded exactly to the query's 16-bit type and stored in
// the same LDS layout, so the products are those of the 16-bit kernel; the
// per-tensor scales fold into the logit scale and the output.  An fp32 cache
// (small workloads) has a plain vector-unit kernel of its own.
#pragma once

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(4))) int* ctab_ptr;   // block table, read-only
typedef const __attribute__((address_space(4))) float* cscale_ptr;   // per-block scales, read-only


// ds_read_b64_tr_b16 at LDS byte address `addr` + OFF.  Issued as inline
// assembly: the compiler treats the builtin as possibly aliasing the LDS-DMA
// copies in flight and would wait for all of them before it.  The result
// may be used only after lds_wait().
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// Wait until at most CNT LDS reads are outstanding (those issued last); the
// values in h are taken as produced here, so no use of them is scheduled
// before the wait.  LDS reads complete in order, and between the reads of a
// batch and this wait no other LDS instruction is issued (the inline
// assembly is ordered against all memory operations).
template <int CNT, int N>
__device__ __forceinline__ void lds_wait(u32x2 (&h)[N]) {
  static_assert(CNT >= 0 && CNT <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(CNT) : "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(h[i]));
}

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
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin

// Tiles are stored row-major (one 2D-byte row per key) with the 16-byte
// chunks of each row XOR-swizzled, so that the LDS reads of the matrix
// operands hit distinct banks:
//  - K operand (ds_read_b128): 16 lanes read one chunk of 16 consecutive
//    rows, so the K swizzle takes a different chunk slot for each of them;
//  - V^T operand (ds_read_b64_tr_b16): lanes read 8-byte pieces of two
//    adjacent chunks of 4 rows per 16-lane group, so the V swizzle moves
//    chunk pairs together (an even XOR) and differs across 8 rows.
// With D = 64 two rows share one 256-byte bank line, hence the row / RPL.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  constexpr int CPR = D / 8, RPL = 256 / (2 * D);
  return (row / RPL) & (CPR - 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  constexpr int CPR = D / 8, RPL = 256 / (2 * D);
  return 2 * ((row / RPL) & (CPR / 2 - 1));
}

// One LDS-DMA load: 16 bytes per lane from `src` to LDS at `dst` + 16 lane.
// (A plain function: target builtins inside templates make the host pass
// drop the kernels' launch stubs.)
__device__ __forceinline__ void dma16(const void* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_char*)dst, 16, 0, 0);
}

// The same through a buffer descriptor: `base` is wave-uniform (it lives in
// scalar registers with the descriptor) and each lane adds its 32-bit byte
// offset `off` < `nbytes`, so no per-lane 64-bit address is formed.
__device__ __forceinline__ void bdma16(const char* base, int nbytes, uint32_t off, char* dst) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_char*)dst, 16, off, 0, 0, 0);
}

// 16 bytes into registers through a buffer descriptor (as bdma16).
__device__ __forceinline__ u32x4 bld16(const char* base, int nbytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nbytes, 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Where a wave's share of a K/V tile comes from.  Wave w copies key rows
// [16 w, 16 w + 16) of every tile, which lie in one cache block (two for
// 8-token blocks), RPI rows (1 KB) per LDS-DMA instruction.  Lane l lands
// at byte 16 l of the instruction's 1 KB, i.e. row l / CPR, chunk slot
// l % CPR, and so fetches the chunk that the swizzle puts there; its byte
// offset inside the block does not change from tile to tile.
template <int D, int BS>
struct TileSrc {
  static constexpr int CPR = D / 8, RPI = 64 / CPR, NI = 16 / RPI, TILE = kKeyTile * D * 2;
  const char* kpool;
  const char* vpool;
  const int* trow;     // the sequence's block-table row
  int64_t head_off;    // byte offset of the KV head inside a block
  int64_t blk_bytes;   // bytes of one block (all heads)
  int kend, wave, lane;
  uint32_t koff[NI], voff[NI];   // this lane's byte offsets inside the block

  __device__ void init(const char* kp, const char* vp, const int* tr, int num_kv_heads, int kvh,
                       int kend_, int wave_, int lane_) {
    kpool = kp;
    vpool = vp;
    trow = tr;
    blk_bytes = (int64_t)num_kv_heads * BS * D * 2;
    head_off = (int64_t)kvh * BS * D * 2;
    kend = kend_;
    wave = wave_;
    lane = lane_;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = 16 * wave + RPI * i + lane / CPR;     // row in the tile
      // row in its block (8-token blocks: the wave's rows lie in two blocks)
      const int brow = BS < 16 ? (RPI * i + lane / CPR) % BS : (16 * wave) % BS + RPI * i + lane / CPR;
      koff[i] = (uint32_t)(brow * D * 2 + 16 * ((lane % CPR) ^ k_swz<D>(row)));
      voff[i] = (uint32_t)(brow * D * 2 + 16 * ((lane % CPR) ^ v_swz<D>(row)));
    }
  }

  // Block ids of this wave's rows in tile kt (scalar loads): rows 0-7 of the
  // wave's 16 in block a, rows 8-15 in block b (the same block unless the
  // block size is 8).
  struct Blk {
    int a, b;
  };
  __device__ __forceinline__ Blk block_of(int kt) const {
    const int key0 = min(kt * kKeyTile + 16 * wave, kend - 1);
    Blk r;
    r.a = ((ctab_ptr)trow)[key0 / BS];
    r.b = BS < 16 ? ((ctab_ptr)trow)[min(key0 + 8, kend - 1) / BS] : r.a;
    return r;
  }

  // Copy this wave's rows of tile kt into a stage (K tile, then V tile);
  // `blk` = block_of(kt).  Keys past the context re-read the last key
  // (finite data; their logits are masked).  Completion is counted by vmcnt.
  __device__ __forceinline__ void copy(int kt, Blk blk, char* dst) const {
    char* kd = dst + 16 * wave * D * 2;
    if (kt * kKeyTile + 16 * wave + 15 < kend) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int bi = (BS < 16 && RPI * i >= 8) ? blk.b : blk.a;   // one block per instruction
        // the KV head's rows of block bi: BS rows of 2 D bytes
        const char* kb = kpool + bi * blk_bytes + head_off;
        const char* vb = vpool + bi * blk_bytes + head_off;
        bdma16(kb, BS * D * 2, koff[i], kd + i * 1024);
        bdma16(vb, BS * D * 2, voff[i], kd + TILE + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = 16 * wave + RPI * i + lane / CPR;
        const int key = min(kt * kKeyTile + row, kend - 1);
        const int64_t base = trow[key / BS] * blk_bytes + head_off + (int64_t)(key % BS) * D * 2;
        dma16(kpool + base + 16 * ((lane % CPR) ^ k_swz<D>(row)), kd + i * 1024);
        dma16(vpool + base + 16 * ((lane % CPR) ^ v_swz<D>(row)), kd + TILE + i * 1024);
      }
    }
  }
};

// 8-bit K/V tiles (fp8 E4M3, or int8 with per-block scales) staged through
// registers.  Thread t of the workgroup owns
// key row t / 4 of every tile and bytes [D/4 (t % 4), D/4 (t % 4 + 1)) of it
// (two 16-byte loads per pool at D = 128, one at D = 64); the 16 rows of a
// wave lie in one cache block (two for 8-token blocks), whose ids come from
// TileSrc::block_of.  store() decodes the codes to T (exact: every E4M3 value
// and every int8 code is a bf16 and an f16 value) and writes them where the
// 16-bit copy would have put them.
template <typename T, int D, int BS, bool I8 = false>
struct TileSrc8 {
  static constexpr int NL = D / 64;             // 16-byte loads per pool and thread
  static constexpr int TILE = kKeyTile * D * 2; // bytes of one 16-bit K or V tile in LDS
  const char* kpool;
  const char* vpool;
  const int* trow;
  int64_t head_off, blk_bytes;                  // in bytes of the 8-bit pools
  int kend, row, sub;
  u32x4 k[NL], v[NL];

  __device__ void init(const char* kp, const char* vp, const int* tr, int num_kv_heads, int kvh, int kend_) {
    kpool = kp;
    vpool = vp;
    trow = tr;
    blk_bytes = (int64_t)num_kv_heads * BS * D;
    head_off = (int64_t)kvh * BS * D;
    kend = kend_;
    row = threadIdx.x >> 2;
    sub = threadIdx.x & 3;
  }

  template <class Blk>
  __device__ __forceinline__ void load(int kt, Blk blk) {
    const int wave_row = row & 15;                      // row among the wave's 16
    if (BS >= 16 && kt * kKeyTile + (row | 15) < kend) {
      // the wave's 16 rows lie in block blk.a: one descriptor per pool (its
      // KV head's BS rows of D bytes), 32-bit offsets per lane
      const char* kb = kpool + blk.a * blk_bytes + head_off;
      const char* vb = vpool + blk.a * blk_bytes + head_off;
      const uint32_t lo = (uint32_t)(((kt * kKeyTile + row) % BS) * D + sub * (D / 4));
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        k[i] = bld16(kb, BS * D, lo + 16 * i);
        v[i] = bld16(vb, BS * D, lo + 16 * i);
      }
      return;
    }
    int64_t off;
    if (kt * kKeyTile + (row | 15) < kend) {
      const int bi = (BS < 16 && wave_row >= 8) ? blk.b : blk.a;
      const int brow = BS < 16 ? wave_row % BS : (kt * kKeyTile + row) % BS;
      off = (int64_t)bi * blk_bytes + head_off + (int64_t)brow * D;
    } else {
      // the wave's rows reach past the context: re-read the last key
      const int key = min(kt * kKeyTile + row, kend - 1);
      off = (int64_t)trow[key / BS] * blk_bytes + head_off + (int64_t)(key % BS) * D;
    }
    off += sub * (D / 4);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      k[i] = ld16(kpool + off + 16 * i);
      v[i] = ld16(vpool + off + 16 * i);
    }
  }

  // Two codes -> a packed pair of T, exactly (fp8 E4M3 or int8 codes).
  static __device__ __forceinline__ uint32_t cvt(uint32_t w, bool hi) {
    if constexpr (I8) return i8x2_to<T>(w, hi);
    else return fp8x2_to<T>(w, hi);
  }

  // Decode and store into a stage (K tile, then V tile).
  __device__ __forceinline__ void store(char* stage) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {        // 8 codes -> one 16-byte chunk of 8 values
        const int chunk = sub * (D / 32) + 2 * i + h;
        const u32x4 kc = {cvt(h ? k[i].z : k[i].x, false), cvt(h ? k[i].z : k[i].x, true),
                          cvt(h ? k[i].w : k[i].y, false), cvt(h ? k[i].w : k[i].y, true)};
        const u32x4 vc = {cvt(h ? v[i].z : v[i].x, false), cvt(h ? v[i].z : v[i].x, true),
                          cvt(h ? v[i].w : v[i].y, false), cvt(h ? v[i].w : v[i].y, true)};
        *reinterpret_cast<u32x4*>(stage + row * D * 2 + 16 * (chunk ^ k_swz<D>(row))) = kc;
        *reinterpret_cast<u32x4*>(stage + TILE + row * D * 2 + 16 * (chunk ^ v_swz<D>(row))) = vc;
      }
    }
  }
};

// Value product of a tile held in the stage at LDS address `stage`:
// acc[b][nb] += V^T(dims 16 nb .., keys) P^T(keys, rows of column tile b),
// and the row sums via the all-ones operand.  For key pair ap (keys 32 ap ..
// 32 ap + 31) the A operand of dimension block nb holds, in lane (G, c16),
// dimension 16 nb + c16 of the lane's eight keys 32 ap + 4 G + 0..3 and
// 32 ap + 16 + 4 G + 0..3 (the probability operand's keys).  A transposing
// read returns to lane c16 of a 16-lane group the element (c16 & 3) of the
// 4-element row addressed by lane 4 t + (c16 >> 2), for t = 0..3; lane s
// therefore addresses key 4 G + (s >> 2) (+ 16 for the second read),
// dimensions 16 nb + 4 (s & 3) .. + 3 (voff).
//
// The reads come in batches of four dimension blocks (eight reads); the
// next batch is in flight while the current one feeds the matrix cores.
template <int D, int AP, int NB0>
__device__ __forceinline__ void pv_read(u32x2 (&h)[8], uint32_t stage, const uint32_t (&voff)[D / 16]) {
  constexpr int OFF0 = 32 * AP * D * 2, OFF1 = (32 * AP + 16) * D * 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[2 * j] = lds_read_tr16<OFF0>(stage + voff[NB0 + j]);
    h[2 * j + 1] = lds_read_tr16<OFF1>(stage + voff[NB0 + j]);
  }
}
template <typename T, int D, int NB0>
__device__ __forceinline__ void pv_mma(f32x4 (&acc)[2][D / 16], const u32x2 (&h)[8], const u32x4 (&pop)[2]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 va = {h[2 * j].x, h[2 * j].y, h[2 * j + 1].x, h[2 * j + 1].y};
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[b][NB0 + j] = PMma<T>::mma(va, pop[b], acc[b][NB0 + j]);
  }
}
// kOnesSum: the row sums of pop are formed here too, as its product with an
// all-ones operand (an int8 cache sums its probabilities on the VALU instead)
template <typename T, int D, bool kOnesSum>
__device__ __forceinline__ void pv_tile(f32x4 (&acc)[2][D / 16], f32x4 (&acc_l)[2], const u32x4 (&pop)[2][2],
                                        uint32_t stage, const uint32_t (&voff)[D / 16]) {
  const u32x4 ones = {kOnes<T>, kOnes<T>, kOnes<T>, kOnes<T>};
  u32x2 h0[8], h1[8];
  if constexpr (D == 128) {
    pv_read<D, 0, 0>(h0, stage, voff);
    pv_read<D, 0, 4>(h1, stage, voff);
    lds_wait<8>(h0);
    pv_mma<T, D, 0>(acc, h0, pop[0]);
    pv_read<D, 1, 0>(h0, stage, voff);
    lds_wait<8>(h1);
    pv_mma<T, D, 4>(acc, h1, pop[0]);
    pv_read<D, 1, 4>(h1, stage, voff);
    lds_wait<8>(h0);
    pv_mma<T, D, 0>(acc, h0, pop[1]);
    lds_wait<0>(h1);
    pv_mma<T, D, 4>(acc, h1, pop[1]);
  } else {
    pv_read<D, 0, 0>(h0, stage, voff);
    pv_read<D, 1, 0>(h1, stage, voff);
    lds_wait<8>(h0);
    pv_mma<T, D, 0>(acc, h0, pop[0]);
    lds_wait<0>(h1);
    pv_mma<T, D, 0>(acc, h1, pop[1]);
  }
  if constexpr (kOnesSum) {
#pragma unroll
    for (int ap = 0; ap < 2; ++ap)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc_l[b] = PMma<T>::mma(ones, pop[ap][b], acc_l[b]);
  }
}

// Work item `lin` of `nwg` (the workgroup's linear index in a launch whose
// workgroups run on XCD lin % kXcds) -> (sequence, KV head, query tile) of a
// grid of nq query tiles x nkv KV heads x sequences.  Each XCD gets a
// contiguous range of work items (query tile fastest), so the query tiles
// that read one (sequence, KV head) context run on the same XCD and share
// its L2.  Longest first: a later query tile sees more keys, and the long
// ones should not be the last to start.  When each XCD's range holds whole
// (sequence, KV head) groups, its workgroups start in order of query tile,
// last tile first, across the groups; otherwise each group's tiles run last
// tile first.
__device__ __forceinline__ void prefill_work(int lin, int nwg, int nq, int nkv, int& seq, int& kvh, int& qtile) {
  const int xq = nwg / kXcds, xr = nwg % kXcds;
  const int xcd = lin % kXcds, slot = lin / kXcds;
  int work;
  if (xr == 0 && xq % nq == 0) {
    const int groups = xq / nq;                      // groups per XCD
    qtile = nq - 1 - slot / groups;
    work = xcd * xq + (slot % groups) * nq + qtile;
  } else {
    work = xcd * xq + min(xcd, xr) + slot;           // a bijection of [0, nwg)
    qtile = nq - 1 - work % nq;
  }
  kvh = (work / nq) % nkv;
  seq = work / (nq * nkv);
}

// One workgroup's query tile: rows qtile * 128 .. of the chunk of sequence
// `seq`, the query heads of KV head `kvh`.
template <typename T, int D, int BS, bool KV8 = false, bool I8 = false>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, int seq, int kvh, int qtile) {
  static_assert(KV8 || !I8, "int8 codes are staged like fp8 codes");
  // an int8 cache's V scale enters the 16-bit probability operand, so with
  // f16 queries the reference max moves with every larger logit (p <= 1)
  constexpr float kSl = (I8 && __is_same(T, _Float16)) ? 0.0f : kSlack;
  extern __shared__ __align__(16) char smem_raw[];
  constexpr int NC = D / 32;
  constexpr int NB = D / 16;                 // 16-dimension blocks of the output
  constexpr int TILE = kKeyTile * D * 2;     // bytes of one K or V tile
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;              // rows per 1 KB DMA instruction
  // stage t (t = 0, 1) at smem_raw + 2 t TILE: K tile, then V tile
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_char*)smem_raw;

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
  const int* trow = p.block_tables + (int64_t)seq * p.max_blocks;

  // the wave index as a wave-uniform value: block ids, copy addresses and the
  // LDS-DMA destinations (M0) derived from it stay in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  // row sums: of the rounded probabilities, formed on the matrix cores by a
  // value product against an all-ones operand (every row of acc_l holds the
  // column's sum), or for an int8 cache of the float32 probabilities, one
  // partial sum per lane in acc_l[b][0] (its four lanes are added at the end).
  float m_run[2] = {-INFINITY, -INFINITY};
  f32x4 acc[2][NB], acc_l[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    acc_l[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nn = 0; nn < NB; ++nn) acc[b][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // first tile that needs the causal mask: every row sees keys <= ctx0 + p0
  const int min_lim = ctx0 + p0;

  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);
  const int ntiles = (kend + kKeyTile - 1) / kKeyTile;

  // LDS byte offsets of this lane's operand pieces inside a stage (the
  // swizzles depend only on the lane, not on the 16-row block or key pair):
  // K piece c of row block a at a * 16 rows + koff[c]; V^T dimension block nb
  // of key pair ap, half hh at (32 ap + 16 hh) rows + voff[nb].
  uint32_t koff[NC], voff[NB];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = c16 * D * 2 + 16 * ((4 * c + G) ^ k_swz<D>(c16));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = 4 * G + (c16 >> 2);
    voff[nb] = TILE + row * D * 2 + 16 * ((2 * nb + ((c16 & 3) >> 1)) ^ v_swz<D>(row)) + 8 * (c16 & 1);
  }

  TileSrc<D, BS> src;
  src.init(kpool, vpool, trow, p.num_kv_heads, kvh, kend, wave, lane);
  TileSrc8<T, D, BS, I8> src8;
  if constexpr (KV8) {
    src8.init(kpool, vpool, trow, p.num_kv_heads, kvh, kend);
    src8.load(0, src.block_of(0));
    src8.store(smem_raw);
  } else {
    src.copy(0, src.block_of(0), smem_raw);
  }
  auto blk_next = src.block_of(1);
  if constexpr (!KV8) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const char* k_lds = smem_raw + (kt & 1) * 2 * TILE;
    const uint32_t v_base = lds_base + (kt & 1) * 2 * TILE;   // LDS address of the stage
    const bool more = kt + 1 < ntiles;     // uniform over the workgroup
    if (more) {
      if constexpr (KV8) src8.load(kt + 1, blk_next);   // into registers
      else src.copy(kt + 1, blk_next, smem_raw + ((kt + 1) & 1) * 2 * TILE);
      blk_next = src.block_of(kt + 2);   // in flight while this tile is computed
    }

    // int8: the K and V scales of the cache block holding this lane's four
    // key rows of each 16-row block (rows 4G .. 4G + 3; the block ids of keys
    // past the context are those of the last key, whose scores are masked)
    float ksc[4], vsc[4];
    if constexpr (I8) {
      const cscale_ptr ksp = (cscale_ptr)p.k_scales, vsp = (cscale_ptr)p.v_scales;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int key = min(kt * kKeyTile + 16 * a + (BS < 16 ? 8 * (G >> 1) : 0), kend - 1);
        const int64_t sidx = (int64_t)((ctab_ptr)trow)[key / BS] * p.num_kv_heads + kvh;
        ksc[a] = ksp[sidx];
        vsc[a] = vsp[sidx];
      }
    }

    // ---- raw products q.k for 4 key row-tiles x 2 query column-tiles
    const bool diag = kt * kKeyTile + kKeyTile - 1 > min_lim;   // uniform
    float s[4][2][4];
    // K pieces of all four 16-key blocks are read up front; the products
    // run c-outermost so that eight independent accumulation chains
    // interleave on the matrix cores.
    u32x4 ka[4][NC];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        ka[a][c] = *reinterpret_cast<const u32x4*>(k_lds + a * 16 * D * 2 + koff[c]);
    // MFMA-heavy phases run at raised wave priority, so that on a SIMD shared
    // with a wave in its softmax phase the matrix core is fed first.
    __builtin_amdgcn_s_setprio(1);
    f32x4 sc[4][2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          sc[a][b] = PMma<T>::mma(ka[a][c], qop[b][c], c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[a][b]);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[a][b][i] = I8 ? sc[a][b][i] * ksc[a] : sc[a][b][i];
    if (diag) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kt * kKeyTile + 16 * a + 4 * G + i > lim[b]) s[a][b][i] = -INFINITY;
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- online softmax per query row (lane column), probabilities -> operands
    // Both column tiles go through each phase together (two independent
    // dependency chains), with one rescaling decision for the pair.
    float mx[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      mx[b] = s[0][b][0];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (a + i > 0) mx[b] = fmax_nan(mx[b], s[a][b][i]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) mx[b] = lanes4_max(mx[b]) * cscale;   // cscale > 0: -inf stays -inf
    // Lazy rescaling (as in decode): the reference max moves only when a
    // row's max exceeds it by more than kSlack, so p <= 2^kSlack; when it
    // moves for some row, every row of the wave takes its exact new max.  A
    // row whose keys are all masked in this tile has mx = -inf and keeps it.
    if (__builtin_amdgcn_ballot_w64(mx[0] > m_run[0] + kSl || mx[1] > m_run[1] + kSl) != 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float m_new = fmaxf(m_run[b], mx[b]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_new);
        m_run[b] = m_new;
        acc_l[b] = acc_l[b] * alpha;
#pragma unroll
        for (int nn = 0; nn < NB; ++nn) acc[b][nn] = acc[b][nn] * alpha;
      }
    }
    // p = 2^(c * (q.k) - m): one fused multiply-add per score.  int8: the
    // value product takes p times the key's block V scale, rounded once, and
    // the row sums add p in float32, so that each weight of the normalised
    // output carries a single rounding.
    u32x4 pop[2][2];   // [key pair][column tile]
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float nm = -m_run[b];
      uint32_t w[4][2];
      float ls = 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[a][b][i], cscale, nm));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[a][b][i + 1], cscale, nm));
          if constexpr (I8) {
            w[a][i / 2] = pack2<T>(e0 * vsc[a], e1 * vsc[a]);
            ls += e0 + e1;
          } else {
            w[a][i / 2] = pack2<T>(e0, e1);
          }
        }
      if constexpr (I8) acc_l[b][0] += ls;
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
        pop[ap][b] = u32x4{w[2 * ap][0], w[2 * ap][1], w[2 * ap + 1][0], w[2 * ap + 1][1]};
    }
    __builtin_amdgcn_s_setprio(1);
    pv_tile<T, D, !I8>(acc, acc_l, pop, v_base, voff);
    __builtin_amdgcn_s_setprio(0);
    if (more) {
      // this wave's copy of the next tile has landed (8-bit: decoded and
      // stored now); after the barrier all copies have, and every wave is
      // done with this tile's stage
      if constexpr (KV8) src8.store(smem_raw + ((kt + 1) & 1) * 2 * TILE);
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

  // ---- normalise and store: lane (G, c16) holds dims 16 nn + 4 G + i of its row
  if constexpr (I8) {
#pragma unroll
    for (int b = 0; b < 2; ++b) acc_l[b][0] = lanes4_sum(acc_l[b][0]);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (!valid[b]) continue;
    const float inv = p.v_scale / acc_l[b][0];
    T* orow = reinterpret_cast<T*>(p.out) +
              ((int64_t)(q0 + pos[b]) * p.num_q_heads + kvh * g + head[b]) * D;
#pragma unroll
    for (int nn = 0; nn < NB; ++nn) {
      const u32x2 w = {pack2<T>(acc[b][nn][0] * inv, acc[b][nn][1] * inv),
                       pack2<T>(acc[b][nn][2] * inv, acc[b][nn][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * nn + 4 * G) = w;
    }
  }
}

}  // namespace pa
