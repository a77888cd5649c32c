// One launch over a mixed serving step: the query tiles of every prefill
// chunk and the decode work of every one-token sequence.
//
// The engine loop the pages describe (ai-engineering page "推理引擎内部机制",
// section "调度器长什么样") forms each step's batch from prefill chunks and
// decodes and runs the step's attention as one fused GPU call.  Here one grid
// holds both kinds of workgroup (four wave64s each).  The first ones are
// decode workgroups running the decode kernel's program on even shares of
// the decode work list; the rest are the prefill query tiles, each running
// the prefill kernel's program.  MI355X dispatches workgroups in index order
// as resources free up, so the decode workgroups spread over the CUs first
// and the prefill tiles fill the other slots: the HBM-bound decode streams
// its K/V beside the matrix-core-bound prefill instead of after it.  How many
// decode workgroups take shares is decided on the device from the step's
// actual sizes (decode bytes against prefill flops) so that both parts end
// together; the surplus ones end at once and their slots take prefill tiles.
// The decode partials that cross workgroup shares are merged by the reduce
// kernel afterwards, as in a decode call.
//
// Each part computes what its own call computes: a prefill tile is the
// prefill kernel's tile program (the same bits as pa_prefill_chunk); the
// decode work is cut by the balanced rule for the decode workgroups that
// take shares, so it may round differently from a pa_decode call.
#include <algorithm>
#include <climits>

#include "decode_dev.h"
#include "prefill_dev.h"

namespace pa {

namespace {

constexpr int kMixedWaves = kPThreads / 64;   // waves per workgroup, both kinds

// Rates of the two kinds of workgroup running side by side on MI355X,
// measured on the mixed workload (16 chunks of 512 tokens over 1,536-token
// contexts beside 112 decodes of 256-4,096 tokens, 32/8 heads, head size
// 128): with a bf16 cache a decode workgroup streams about 24.5 KB of K/V
// per microsecond and a prefill slot does about 1.34 Mflop per microsecond.
// [1] is the fp8 E4M3 cache: the decode rate scaled by the fp8 decode
// kernel's byte rate against the bf16 one, the prefill rate by the fp8
// prefill tiles' (codes decoded into LDS through registers); on that
// workload over an fp8 cache any split from 96 to 256 decode workgroups
// lands within 2 % of the best.  [2], the int8 cache with per-block scales:
// on the 70B-shaped int8 serving step (4 chunks of 512 tokens, 128 decodes,
// 64/8 heads, block 16) a decode rate of 19 KB/us beside 1.25 Mflop/us gave
// the shortest launch among 16-29 KB/us (1-5 % apart).  Only the
// ratio of a pair matters; it sets how many slots the decode part takes.
constexpr double kDecodeWgBytesPerUs[3] = {24.5e3, 21.2e3, 19.0e3};
constexpr double kPrefillSlotFlopsPerUs[3] = {1.34e6, 1.30e6, 1.25e6};

// Sum over the workgroup (every thread gets it); ends with a barrier.
__device__ __forceinline__ double wg_sum(double v) {
  __shared__ double part[kMixedWaves];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kMixedWaves; ++w) t += part[w];
  __syncthreads();
  return t;
}

// Decode workgroups that take shares, from the step's actual sizes: the
// decode's K/V bytes (from the clamped lengths of the plan) and the prefill's
// visible (query, key) pairs (from the chunk offsets and context lengths).
// The decode part gets the share of the resident slots that lets both parts
// end together: ndec / (slots - ndec) = (decode workgroup-time needed) /
// (prefill slot-time needed).  Every decode workgroup computes the same
// count from the same data.
struct MixedPick {
  const int* query_start_loc;
  const int* prefill_lens;
  int num_chunks, cap;          // cap: longest context a prefill table row holds
  int num_q_heads, num_kv_heads, head_dim, elem_bytes, slots;
  double decode_rate, prefill_rate;   // bytes per µs per decode workgroup, flops per µs per prefill slot
  __device__ int operator()(const int* lens, int S, int nwg) const {
    double units = 0.0, pairs = 0.0;
    for (int s = threadIdx.x; s < S; s += kPThreads) units += (double)((lens[s] + 31) / 32);
    for (int s = threadIdx.x; s < num_chunks; s += kPThreads) {
      const int L = query_start_loc[s + 1] - query_start_loc[s];
      const int n = min(prefill_lens[s], cap);
      if (L > 0 && n >= L) pairs += (double)L * (n - L) + 0.5 * (double)L * (L + 1);
    }
    units = wg_sum(units);
    pairs = wg_sum(pairs);
    if (pairs <= 0.0) return nwg;                  // no prefill work: every slot decodes
    const double bytes = units * 32.0 * num_kv_heads * head_dim * 2.0 * elem_bytes;
    const double flops = 4.0 * head_dim * num_q_heads * pairs;
    const double k = (bytes / decode_rate) / (flops / prefill_rate);
    int n = (int)fmin((double)nwg, ceil((double)slots * k / (1.0 + k)));
    n = (n + kXcds - 1) / kXcds * kXcds;           // whole rounds over the XCDs
    return n < kXcds ? kXcds : (n > nwg ? nwg : n);
  }
};

// Cache formats of the mixed step: the query type, fp8 E4M3 codes, int8
// codes with per-(block, KV head) scales.
enum : int { kMixQ = 0, kMixFp8 = 1, kMixI8 = 2 };

// The decode program of a cache format.
template <typename T, int D, int BS, int FMT>
using MixedSeg = MfmaDecode<T, FMT == kMixFp8 ? kFmtFp8 : (FMT == kMixI8 ? kFmtI8 : kFmtQ),
                            FMT == kMixFp8 ? kFmtFp8 : (FMT == kMixI8 ? kFmtI8 : kFmtQ), D, BS>;

template <typename T, int D, int BS, int FMT>
__global__ __launch_bounds__(kPThreads) void mixed_kernel(PrefillParams pf, DecodeParams d, int npf, int ndec,
                                                          int nq, int slots) {
  const int b = blockIdx.x;
  if (b < ndec) {
    const MixedPick pick{pf.query_start_loc, pf.seq_lens, npf > 0 ? pf.num_seqs : 0, pf.max_blocks * BS,
                         d.num_q_heads, d.num_kv_heads, D, FMT == kMixQ ? (int)sizeof(T) : 1, slots,
                         kDecodeWgBytesPerUs[FMT], kPrefillSlotFlopsPerUs[FMT]};
    decode_share<MixedSeg<T, D, BS, FMT>, T, kMixedWaves>(d, b, ndec, pick);
    return;
  }
  // ndec is a multiple of the XCD count, so tile lin runs on XCD lin % kXcds
  // as in a prefill launch
  int seq, kvh, qtile;
  prefill_work(b - ndec, npf, nq, pf.num_kv_heads, seq, kvh, qtile);
  prefill_tile<T, D, BS, FMT != kMixQ, FMT == kMixI8>(pf, seq, kvh, qtile);
}

template <typename T, int D, int BS, int FMT>
hipError_t launch_mixed_t(const PrefillParams& pf, const DecodeParams& d0, hipStream_t stream) {
  auto kernel = mixed_kernel<T, D, BS, FMT>;
  DecodeParams d = d0;
  const int qpos = pf.num_seqs > 0 ? kRowsPerWG / pf.group : 1;   // chunk positions per tile
  const int nq = (pf.num_seqs > 0 && pf.max_q_len > 0) ? (pf.max_q_len + qpos - 1) / qpos : 0;
  const int64_t npf = (int64_t)nq * pf.num_kv_heads * pf.num_seqs;
  // LDS: the prefill tile's two K/V stages; a decode workgroup's plan,
  // merge slots (up to three per wave) and, for 8-bit K, each wave's 4 KB K
  // staging fit in the same bytes
  const size_t stages = prefill_smem_bytes(D);
  size_t lds = npf > 0 ? stages : 0;
  d.local_slots = 0;
  if (d.num_seqs > 0) {
    const size_t plan = (size_t)((2 * d.num_seqs + 1 + 3) & ~3) * sizeof(int);
    const size_t per_slot = (size_t)d.group * D * sizeof(float) + 33 * sizeof(float);
    const size_t kstage = MixedSeg<T, D, BS, FMT>::kStageK ? (size_t)kMixedWaves * 4096 : 0;
    const size_t room = stages > plan + 64 + kstage ? stages - kstage : plan + 64;
    int slots = 0;
    if (d.mode != kSplitNone && plan + 64 < room)
      slots = (int)std::min<size_t>((size_t)3 * kMixedWaves, (room - plan - 64) / per_slot);
    d.local_slots = slots;
    const size_t merge_end = plan + (size_t)((slots + 3) & ~3) * sizeof(int) + (size_t)slots * 32 * sizeof(float) +
                             (size_t)slots * d.group * D * sizeof(float);
    d.kstage_off = (int)merge_end;
    lds = lds > merge_end + kstage ? lds : merge_end + kstage;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), kPThreads,
                                                   lds) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  // Decode workgroups, all dispatched first so that they spread over the
  // CUs beside the first prefill tiles: one per resident slot (no more than
  // have work, whole rounds over the XCDs), of which the count MixedPick
  // computes on the device take shares and the rest end at once.
  const int64_t slots = (int64_t)cu_count() * per_cu;
  int64_t ndec = 0;
  if (d.num_seqs > 0) {
    ndec = slots;
    const int64_t need = (wave_work_bound(d) + kMixedWaves - 1) / kMixedWaves;
    if (ndec > need) ndec = need;
    ndec = (ndec + kXcds - 1) / kXcds * kXcds;
  }
  const int64_t grid = npf + ndec;
  if (grid == 0) return hipSuccess;
  if (grid > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kPThreads), lds, stream, pf, d, (int)npf, (int)ndec, nq,
                     (int)slots);
  return hipGetLastError();
}

template <typename T, int D, int FMT>
hipError_t launch_mixed_bs(const PrefillParams& pf, const DecodeParams& d, int block_size, hipStream_t s) {
  switch (block_size) {
    case 8: return launch_mixed_t<T, D, 8, FMT>(pf, d, s);
    case 16: return launch_mixed_t<T, D, 16, FMT>(pf, d, s);
    case 32: return launch_mixed_t<T, D, 32, FMT>(pf, d, s);
    default: return launch_mixed_t<T, D, 64, FMT>(pf, d, s);
  }
}

template <typename T, int FMT>
hipError_t launch_mixed_f(const PrefillParams& pf, const DecodeParams& d, int head_dim, int block_size,
                          hipStream_t s) {
  if (head_dim == 128) return launch_mixed_bs<T, 128, FMT>(pf, d, block_size, s);
  return launch_mixed_bs<T, 64, FMT>(pf, d, block_size, s);
}

template <typename T>
hipError_t launch_mixed_d(const PrefillParams& pf, const DecodeParams& d, int head_dim, int block_size, int fmt,
                          hipStream_t s) {
  if (fmt == kMixFp8) return launch_mixed_f<T, kMixFp8>(pf, d, head_dim, block_size, s);
  if (fmt == kMixI8) return launch_mixed_f<T, kMixI8>(pf, d, head_dim, block_size, s);
  return launch_mixed_f<T, kMixQ>(pf, d, head_dim, block_size, s);
}

}  // namespace

hipError_t launch_mixed(const PrefillParams& pf, const DecodeParams& d, hipStream_t stream) {
  const bool has_pf = pf.num_seqs > 0, has_d = d.num_seqs > 0;
  if (!has_pf && !has_d) return hipSuccess;
  // K and V pools of the query type, or both fp8, or both int8 with block
  // scales; with both parts present they share the pools, the head shape and
  // the block size
  const auto pool_ok = [](int q, int c) { return c == q || c == kFP8 || c == kI8; };
  if (has_pf && (!pool_ok(pf.q_dtype, pf.cache_dtype) || (pf.cache_dtype == kI8 && !pf.k_scales)))
    return hipErrorInvalidValue;
  if (has_d && (d.v_cache_dtype != d.cache_dtype || !pool_ok(d.q_dtype, d.cache_dtype) ||
                (d.cache_dtype == kI8 && !d.k_scales)))
    return hipErrorInvalidValue;
  if (has_pf && has_d &&
      (pf.head_dim != d.head_dim || pf.block_size != d.block_size || pf.num_kv_heads != d.num_kv_heads ||
       pf.group != d.group || pf.q_dtype != d.q_dtype || pf.cache_dtype != d.cache_dtype))
    return hipErrorInvalidValue;
  const int q_dtype = has_d ? d.q_dtype : pf.q_dtype;
  const int head_dim = has_d ? d.head_dim : pf.head_dim;
  const int block_size = has_d ? d.block_size : pf.block_size;
  const int cache = has_d ? d.cache_dtype : pf.cache_dtype;
  const int fmt = cache == kFP8 ? kMixFp8 : (cache == kI8 ? kMixI8 : kMixQ);
  if (q_dtype == kBF16) return launch_mixed_d<__bf16>(pf, d, head_dim, block_size, fmt, stream);
  if (q_dtype == kF16) return launch_mixed_d<_Float16>(pf, d, head_dim, block_size, fmt, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
