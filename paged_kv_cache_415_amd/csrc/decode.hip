// Paged decode attention on gfx950: the persistent decode kernel, the
// log-sum-exp reduce of split partials and their launchers.  The device code
// of a workgroup's share (plan, work list, segments) is in decode_dev.h.
#include <mutex>

#include "decode_dev.h"

namespace pa {

// The persistent kernel: one workgroup per CU holding all the waves the CU
// keeps resident.
template <class Seg, typename QT>
__global__ __launch_bounds__(Seg::kWaves * 64) void decode_kernel(DecodeParams p) {
  decode_share<Seg, QT, Seg::kWaves>(p, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials of one (sequence, query head):
//   M = max_i m_i,  out = v_scale * sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i
// One wave per query head (four per workgroup): lane i takes partial i's
// weight; the dims of the output are spread over the lanes.  The partial
// rows are read eight at a time, the first eight together with m and l, so
// a head costs two dependent memory round trips (its count, then the rest).
// The attention kernel stores a count for every pair: 0 for an empty
// sequence, 1 for a pair whose output it stored itself (one segment, or
// partials merged on the CU).
// ---------------------------------------------------------------------------
template <int E>
__device__ __forceinline__ void load_rows8(const float* po, int D, int first, int last, float (&x)[8][E]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t row = min(first + u, last);   // rows past the last are re-read, weight 0
    if constexpr (E == 2) {
      const float2 v = *reinterpret_cast<const float2*>(po + row * D);
      x[u][0] = v.x;
      x[u][1] = v.y;
    } else {
      x[u][0] = po[row * D];
    }
  }
}

template <int E>
__device__ __forceinline__ void accum_rows8(float w, int t, const float (&x)[8][E], float (&O)[E]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    // lane t + u <= 63 holds that partial's weight (0 past the count)
    const float wf = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), t + u));
#pragma unroll
    for (int e = 0; e < E; ++e) O[e] += wf * x[u][e];
  }
}

template <typename QT, int D>
__global__ __launch_bounds__(256) void lse_reduce_kernel(DecodeParams p) {
  constexpr int E = D / 64;   // output dims per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hq = blockIdx.x * 4 + wave, s = blockIdx.y;
  if (hq >= p.num_q_heads) return;
  const int np = p.nparts[s * p.num_kv_heads + hq / p.group];
  if (np <= 1) return;
  const int64_t b = ((int64_t)s * p.num_q_heads + hq) * p.max_parts;
  const float* pm = p.part_m + b;
  const float* pl = p.part_l + b;
  const float* po = p.part_o + b * D + E * lane;

  const int n0 = min(64, np);
  float x[8][E];
  load_rows8<E>(po, D, 0, n0 - 1, x);
  const float m0 = lane < n0 ? pm[lane] : -INFINITY;
  const float l0 = lane < n0 ? pl[lane] : 0.f;
  float M = m0;
  for (int i = 64 + lane; i < np; i += 64) M = fmaxf(M, pm[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));

  float O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  // Sums run over the partials in order (the weights from lane t), the same
  // arithmetic as the attention kernel's merge of partials it keeps in LDS,
  // so both give the same bits.
  float w = lane < n0 ? __builtin_amdgcn_exp2f(m0 - M) : 0.f;
  float L = 0.f;
  for (int t = 0; t < n0; ++t)
    L += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), t)) *
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l0), t));
  accum_rows8<E>(w, 0, x, O);
  for (int t = 8; t < n0; t += 8) {
    load_rows8<E>(po, D, t, n0 - 1, x);
    accum_rows8<E>(w, t, x, O);
  }
  for (int c = 64; c < np; c += 64) {
    const int n = min(64, np - c);
    w = lane < n ? __builtin_amdgcn_exp2f(pm[c + lane] - M) : 0.f;
    const float lc = lane < n ? pl[c + lane] : 0.f;
    for (int t = 0; t < n; ++t)
      L += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), t)) *
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lc), t));
    for (int t = 0; t < n; t += 8) {
      load_rows8<E>(po, D, c + t, c + n - 1, x);
      accum_rows8<E>(w, t, x, O);
    }
  }
  const float inv = p.v_scale / L;
  QT* orow = reinterpret_cast<QT*>(p.out) + ((int64_t)s * p.num_q_heads + hq) * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[e] = (QT)(O[e] * inv);
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
size_t decode_plan_lds_bytes(int num_seqs) { return (size_t)(2 * num_seqs + 1) * sizeof(int); }
int decode_max_plan_seqs() { return kMaxPlanSeqs; }

namespace {
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];
}  // namespace

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  });
  return g_cu_count[dev];
}

// Upper bound of the waves that can have work, from host-known sizes.
int64_t wave_work_bound(const DecodeParams& p) {
  const int64_t umax = (p.max_len + kStep - 1) / kStep;
  const int64_t pairs = (int64_t)p.num_seqs * p.num_kv_heads;
  if (p.mode == kSplitBalanced) return (pairs * umax + p.chunk - 1) / p.chunk;
  if (p.mode == kSplitNone) return pairs;
  return pairs * ((umax + p.chunk - 1) / p.chunk);
}

namespace {

int g_lds_max[kMaxDevices];
std::once_flag g_lds_once[kMaxDevices];

// Dynamic LDS a decode workgroup may take: the device's per-workgroup limit
// less 8 KB (static LDS and margin), at most 150 KB.
size_t lds_budget() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 56 * 1024;
  std::call_once(g_lds_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || n <= 0)
      n = 64 * 1024;
    g_lds_max[dev] = n;
  });
  return std::min<size_t>(150 * 1024, (size_t)g_lds_max[dev] - 8 * 1024);
}

template <class Seg, typename QT>
hipError_t launch_persistent(const DecodeParams& p0, hipStream_t stream) {
  constexpr int NT = 64 * Seg::kWaves;
  DecodeParams p = p0;
  // LDS: the plan, then as many merge slots as fit (up to three per wave)
  const size_t plan = (size_t)((2 * p.num_seqs + 1 + 3) & ~3) * sizeof(int);
  const size_t per_slot = (size_t)p.group * p.head_dim * sizeof(float) + 33 * sizeof(float);
  const size_t stage = Seg::kStageK ? (size_t)Seg::kWaves * 4096 : 0;   // 8-bit K staging
  const size_t budget = lds_budget() - stage;
  int slots = 0;
  if (Seg::kLocalMerge && p.mode != kSplitNone && plan + 64 < budget)
    slots = (int)std::min<size_t>((size_t)3 * Seg::kWaves, (budget - plan - 64) / per_slot);
  p.local_slots = slots;
  const size_t merge_end = plan + (size_t)((slots + 3) & ~3) * sizeof(int) + (size_t)slots * 32 * sizeof(float) +
                           (size_t)slots * p.group * p.head_dim * sizeof(float);
  p.kstage_off = (int)merge_end;
  const size_t lds = merge_end + stage;
  auto kernel = decode_kernel<Seg, QT>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), NT,
                                                   lds) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  int64_t grid = (int64_t)cu_count() * per_cu;
  const int64_t need = (wave_work_bound(p) + Seg::kWaves - 1) / Seg::kWaves;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NT), lds, stream, p);
  return hipGetLastError();
}

template <typename QT, int KF, int VF, int D, bool APPEND = false>
hipError_t launch_mfma_bs(const DecodeParams& p, hipStream_t s) {
  switch (p.block_size) {
    case 8: return launch_persistent<MfmaDecode<QT, KF, VF, D, 8, APPEND>, QT>(p, s);
    case 16: return launch_persistent<MfmaDecode<QT, KF, VF, D, 16, APPEND>, QT>(p, s);
    case 32: return launch_persistent<MfmaDecode<QT, KF, VF, D, 32, APPEND>, QT>(p, s);
    default: return launch_persistent<MfmaDecode<QT, KF, VF, D, 64, APPEND>, QT>(p, s);
  }
}

template <int D>
hipError_t launch_f32_bs(const DecodeParams& p, hipStream_t s) {
  switch (p.block_size) {
    case 8: return launch_persistent<F32Decode<D, 8>, float>(p, s);
    case 16: return launch_persistent<F32Decode<D, 16>, float>(p, s);
    case 32: return launch_persistent<F32Decode<D, 32>, float>(p, s);
    default: return launch_persistent<F32Decode<D, 64>, float>(p, s);
  }
}

template <typename QT, int KF, int VF, bool APPEND = false>
hipError_t launch_mfma(const DecodeParams& p, hipStream_t s) {
  if (p.head_dim == 128) return launch_mfma_bs<QT, KF, VF, 128, APPEND>(p, s);
  return launch_mfma_bs<QT, KF, VF, 64, APPEND>(p, s);
}

template <typename QT>
hipError_t launch_mfma_formats(const DecodeParams& p, hipStream_t s) {
  if (p.new_k != nullptr) return launch_mfma<QT, kFmtQ, kFmtQ, true>(p, s);
  if (p.cache_dtype == kI8) return launch_mfma<QT, kFmtI8, kFmtI8>(p, s);
  const bool kf8 = p.cache_dtype == kFP8, vf8 = p.v_cache_dtype == kFP8;
  if (kf8 && vf8) return launch_mfma<QT, kFmtFp8, kFmtFp8>(p, s);
  if (kf8) return launch_mfma<QT, kFmtFp8, kFmtQ>(p, s);
  return launch_mfma<QT, kFmtQ, kFmtQ>(p, s);
}

}  // namespace

hipError_t launch_decode_attention(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  if (p.cache_dtype == kF32) return p.head_dim == 128 ? launch_f32_bs<128>(p, stream) : launch_f32_bs<64>(p, stream);
  if (p.q_dtype == kBF16) return launch_mfma_formats<__bf16>(p, stream);
  return launch_mfma_formats<_Float16>(p, stream);
}

namespace {

template <int D>
void launch_reduce_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((p.num_q_heads + 3) / 4, p.num_seqs);
  if (p.q_dtype == kF32)
    hipLaunchKernelGGL((lse_reduce_kernel<float, D>), grid, dim3(256), 0, stream, p);
  else if (p.q_dtype == kBF16)
    hipLaunchKernelGGL((lse_reduce_kernel<__bf16, D>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((lse_reduce_kernel<_Float16, D>), grid, dim3(256), 0, stream, p);
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0 || p.mode == kSplitNone) return hipSuccess;
  if (p.head_dim == 128) launch_reduce_d<128>(p, stream);
  else launch_reduce_d<64>(p, stream);
  return hipGetLastError();
}

}  // namespace pa
