// Top-k gating and dispatch metadata on the device.
//
// The routing metadata (counts, offsets, the packed row of every routed slot) is built
// and kept on the GPU so the host can enqueue the expert GEMMs without waiting for a
// copy-back (unite.ai, "Ai2 κυκλοφορεί το Olmo-Core 3…", section "Παραλληλισμός,
// Ακρίβεια και Τεχνικές Μνήμης"; ettayeb.fr, "Olmo-core 3 ouvre l'entraînement des
// MoE…", section "Trois parallélismes, trois optimisations de routage").
//
// Three launches, all with host-known grids:
//   1. per chunk of 32 tokens (16 waves, two tokens each): wave-level top-k of each
//      token's E scores, its gates, and
//      a stable in-chunk rank of every routed slot (ballot matching) plus the chunk's
//      per-expert histogram;
//   2. one workgroup: per-expert running sums over chunks (chunk bases), counts, and the
//      exclusive prefix sum over experts (offsets);
//   3. per slot: slot_row = offsets[e] + chunk base + in-chunk rank.
// The result is the stable counting sort of slots t*k + j by expert, bit for bit.
#include <mutex>

#include "common.h"
#include "gemm.h"
#include "route.h"

// Fixed scratch of the allocation-free routing entry point: the per-chunk expert histograms
// and in-chunk ranks that route_topk otherwise keeps in the caller's workspace.  Each GPU the
// library runs on holds its own copy for the life of the process.  Host code never names it
// directly (the name is a host-side stand-in, not a device address): it uses the per-device
// address that route_scratch_ptr() takes with hipGetSymbolAddress.
static __device__ __align__(256) int32_t scratch[moe::kRouteScratchInts];

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
int32_t* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// 16 waves per chunk, two tokens each: the per-token top-k is a chain of dependent
// cross-lane reductions, so many waves per compute unit keep it fed
constexpr int kThreads = 1024;
constexpr int kTokPerWave = kRouteChunk / (kThreads / kWave);
static_assert(kTokPerWave * (kThreads / kWave) == kRouteChunk, "whole tokens per wave");

// (value desc, index asc) total order on (score, expert)
__device__ __forceinline__ bool beats(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <int EPL, bool GIVEN>
__global__ void __launch_bounds__(kThreads) route_chunk_kernel(int T, int E, int k, const float* __restrict__ logits,
                                                               const int32_t* __restrict__ given_idx,
                                                               int32_t* __restrict__ topk_idx, float* __restrict__ gates,
                                                               int32_t* __restrict__ hist, int32_t* __restrict__ local_rank,
                                                               int32_t* __restrict__ dev_err) {
  __shared__ int s_sel[kRouteChunk * kMaxTopK];
  __shared__ int s_cnt[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x;
  const int t0 = chunk * kRouteChunk;
  for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;

  for (int q = 0; q < kTokPerWave; q++) {
    const int tl = wave * kTokPerWave + q;
    const int t = t0 + tl;
    if (t >= T) break;
    if constexpr (!GIVEN) {
      float v[EPL];
#pragma unroll
      for (int i = 0; i < EPL; i++) {
        const int e = lane + kWave * i;
        v[i] = e < E ? logits[(int64_t)t * E + e] : 0.f;
      }
      uint32_t taken = 0;
      float top_v = 0.f, sum = 0.f, first = 0.f;
      for (int j = 0; j < k; j++) {
        float bv = 0.f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; i++) {
          const int e = lane + kWave * i;
          if (e < E && !((taken >> i) & 1u) && (bi == 0x7fffffff || beats(v[i], e, bv, bi))) { bv = v[i]; bi = e; }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ov = __shfl_xor(bv, o, kWave);
          const int oi = __shfl_xor(bi, o, kWave);
          if (oi != 0x7fffffff && (bi == 0x7fffffff || beats(ov, oi, bv, bi))) { bv = ov; bi = oi; }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (j == 0) first = bv;
        const float w = expf(bv - first);
        sum += w;
        if (lane == j) { top_v = w; s_sel[tl * k + j] = bi; topk_idx[(int64_t)t * k + j] = bi; }
      }
      if (lane < k) gates[(int64_t)t * k + lane] = top_v / sum;
    } else {
      if (lane < k) {
        int e = given_idx[(int64_t)t * k + lane];
        int err = 0;
        if (e < 0 || e >= E) { err |= MOE_DEVERR_EXPERT_RANGE_BIT; e = e < 0 ? 0 : E - 1; }
        for (int j = 0; j < lane; j++) {
          int o = given_idx[(int64_t)t * k + j];
          o = o < 0 ? 0 : (o >= E ? E - 1 : o);
          if (o == e) err |= MOE_DEVERR_DUPLICATE_BIT;
        }
        if (err) atomicOr(dev_err, err);
        s_sel[tl * k + lane] = e;
      }
    }
  }
  __syncthreads();

  // stable in-chunk rank: wave 0 walks the chunk's slots in order, 64 at a time
  if (wave == 0) {
    const int ntok = min(kRouteChunk, T - t0);
    const int nslots = ntok * k;
    int nbits = 1;
    while ((1 << nbits) < E) nbits++;
    for (int base = 0; base < nslots; base += kWave) {
      const int s = base + lane;
      const bool valid = s < nslots;
      const int e = valid ? s_sel[s] : 0;
      uint64_t mask = __ballot(valid);
      for (int b = 0; b < nbits; b++) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(valid && bit);
        mask &= bit ? bal : ~bal;
      }
      const uint64_t lower = mask & ((1ull << lane) - 1ull);
      int rank = 0;
      if (valid) rank = s_cnt[e] + __popcll(lower);
      __builtin_amdgcn_wave_barrier();
      const bool last = valid && ((mask >> lane) >> 1) == 0;  // highest lane of its expert group
      if (last) s_cnt[e] = rank + 1;
      __builtin_amdgcn_wave_barrier();
      if (valid) local_rank[(int64_t)t0 * k + s] = rank;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) hist[(int64_t)chunk * E + e] = s_cnt[e];
}

// One workgroup: chunk bases (exclusive running sums over chunks, in place over the
// histograms), counts and offsets.  The chunks are split into P contiguous runs (P a power
// of two, P * E <= 1024); thread (part, expert) = (tid / E, tid % E) walks one run of one
// expert, so a wave's loads read consecutive experts of one chunk row.  Every thread sums
// its run, the sums meet in LDS, and each thread rewrites its run with the running bases.
__global__ void __launch_bounds__(1024) route_scan_kernel(int E, int nchunks, int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int s_wave[16];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_part[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int P = 1;
  while (P < kWave && 2 * P * E <= 1024) P *= 2;
  const int part = tid / E, ex = tid - part * E;
  const bool active = part < P;
  const int c0 = active ? (int)((int64_t)part * nchunks / P) : 0;
  const int c1 = active ? (int)((int64_t)(part + 1) * nchunks / P) : 0;
  // a run of at most kScanHeld chunks is loaded once, every load issued before the first
  // add, and kept in registers for the rewrite; longer runs are read twice
  constexpr int kScanHeld = 64;
  const int n = c1 - c0;
  const bool held = n <= kScanHeld;
  int v[kScanHeld];
  int sum = 0;
  if (held) {
#pragma unroll
    for (int i = 0; i < kScanHeld; i++) v[i] = i < n ? hist[(int64_t)(c0 + i) * E + ex] : 0;
#pragma unroll
    for (int i = 0; i < kScanHeld; i++) sum += v[i];
  } else {
#pragma unroll 8
    for (int c = c0; c < c1; c++) sum += hist[(int64_t)c * E + ex];
  }
  if (active) s_part[tid] = sum;
  __syncthreads();
  if (active) {
    int run = 0;
    for (int q = 0; q < part; q++) run += s_part[q * E + ex];
    if (held) {
#pragma unroll
      for (int i = 0; i < kScanHeld; i++) {
        if (i < n) hist[(int64_t)(c0 + i) * E + ex] = run;
        run += v[i];
      }
    } else {
#pragma unroll 8
      for (int c = c0; c < c1; c++) {
        const int h = hist[(int64_t)c * E + ex];
        hist[(int64_t)c * E + ex] = run;
        run += h;
      }
    }
    if (part == P - 1) s_cnt[ex] = run;
  }
  __syncthreads();
  const int run = tid < E ? s_cnt[tid] : 0;
  if (tid < E) counts[tid] = run;
  // exclusive scan of the counts over experts
  int incl = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int carry = 0;
  for (int w = 0; w < wave; w++) carry += s_wave[w];
  if (tid < E) offsets[tid] = carry + incl - run;
  if (tid == E - 1) offsets[E] = carry + incl;
}

__global__ void route_finalize_kernel(int T, int E, int k, const int32_t* __restrict__ idx,
                                      const int32_t* __restrict__ hist, const int32_t* __restrict__ local_rank,
                                      const int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= (int64_t)T * k) return;
  int e = idx[s];
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const int chunk = (int)(s / k) / kRouteChunk;
  slot_row[s] = offsets[e] + hist[(int64_t)chunk * E + e] + local_rank[s];
}

// dlogits[t, e] = g_e (dg_e - sum_i g_i dg_i) on the chosen experts, else 0.  A thread
// writes four consecutive experts of one token (one 16-byte store when VEC: E % 4 == 0 and
// dlogits 16-byte aligned), so each token's k gates, gate gradients and expert ids are
// read by E / 4 threads instead of E.
template <bool VEC>
__global__ void route_bwd_kernel(int T, int E, int k, const float* __restrict__ dgates, const float* __restrict__ gates,
                                 const int32_t* __restrict__ idx, float* __restrict__ dlogits) {
  const int E4 = (E + 3) / 4;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= (int64_t)T * E4) return;
  const int t = (int)(q / E4), e0 = (int)(q % E4) * 4;
  const float* g = gates + (int64_t)t * k;
  const float* dg = dgates + (int64_t)t * k;
  const int32_t* id = idx + (int64_t)t * k;
  float inner = 0.f;
  for (int j = 0; j < k; j++) inner = fmaf(g[j], dg[j], inner);
  float out[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; j++) {
    const int r = id[j] - e0;
#pragma unroll
    for (int c = 0; c < 4; c++)
      if (r == c) out[c] = g[j] * (dg[j] - inner);
  }
  float* o = dlogits + (int64_t)t * E + e0;
  if constexpr (VEC) {
    *reinterpret_cast<float4*>(o) = make_float4(out[0], out[1], out[2], out[3]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; c++)
      if (e0 + c < E) o[c] = out[c];
  }
}

template <bool GIVEN>
hipError_t launch_chunk(int T, int E, int k, const float* logits, const int32_t* given, int32_t* idx, float* gates,
                        int32_t* hist, int32_t* rank, int32_t* dev_err, hipStream_t st) {
  const int nchunks = (T + kRouteChunk - 1) / kRouteChunk;
  const int epl = (E + kWave - 1) / kWave;
#define MOE_ROUTE_CASE(N)                                                                                   \
  if (epl <= N) {                                                                                           \
    hipLaunchKernelGGL((route_chunk_kernel<N, GIVEN>), dim3(nchunks), dim3(kThreads), 0, st, T, E, k, logits, \
                       given, idx, gates, hist, rank, dev_err);                                              \
    return hipGetLastError();                                                                               \
  }
  MOE_ROUTE_CASE(1) MOE_ROUTE_CASE(2) MOE_ROUTE_CASE(4) MOE_ROUTE_CASE(8) MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

size_t route_workspace_bytes(int T, int E, int k) {
  const size_t nchunks = (size_t)(T + kRouteChunk - 1) / kRouteChunk;
  return (nchunks * E + (size_t)T * k) * sizeof(int32_t);
}

// Device address of `scratch` on the current device, taken once per device (with that
// device current) and kept.
hipError_t route_scratch_ptr(int32_t** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t route_topk(int T, int E, int k, const float* logits, int32_t* idx, float* gates, int32_t* counts,
                      int32_t* offsets, int32_t* slot_row, void* ws, hipStream_t st) {
  const int nchunks = (T + kRouteChunk - 1) / kRouteChunk;
  int32_t* hist = static_cast<int32_t*>(ws);
  int32_t* rank = hist + (size_t)nchunks * E;
  hipError_t err = hipSuccess;
  if (nchunks > 0 && (err = launch_chunk<false>(T, E, k, logits, nullptr, idx, gates, hist, rank, nullptr, st)) != hipSuccess)
    return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, st, E, nchunks, hist, counts, offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t S = (int64_t)T * k;
  if (S == 0) return hipSuccess;
  hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)((S + 255) / 256)), dim3(256), 0, st, T, E, k, idx, hist,
                     rank, offsets, slot_row);
  return hipGetLastError();
}

hipError_t route_given(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                       int32_t* slot_row, int32_t* dev_err, void* ws, hipStream_t st) {
  const int nchunks = (T + kRouteChunk - 1) / kRouteChunk;
  int32_t* hist = static_cast<int32_t*>(ws);
  int32_t* rank = hist + (size_t)nchunks * E;
  hipError_t err = hipSuccess;
  if (nchunks > 0 && (err = launch_chunk<true>(T, E, k, nullptr, idx, nullptr, nullptr, hist, rank, dev_err, st)) != hipSuccess)
    return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, st, E, nchunks, hist, counts, offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t S = (int64_t)T * k;
  if (S == 0) return hipSuccess;
  hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)((S + 255) / 256)), dim3(256), 0, st, T, E, k, idx, hist,
                     rank, offsets, slot_row);
  return hipGetLastError();
}

hipError_t route_backward(int T, int E, int k, const float* dgates, const float* gates, const int32_t* idx,
                          float* dlogits, hipStream_t st) {
  const int64_t n = (int64_t)T * ((E + 3) / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (E % 4 == 0 && (reinterpret_cast<uintptr_t>(dlogits) & 15) == 0)
    hipLaunchKernelGGL(route_bwd_kernel<true>, grid, dim3(256), 0, st, T, E, k, dgates, gates, idx, dlogits);
  else
    hipLaunchKernelGGL(route_bwd_kernel<false>, grid, dim3(256), 0, st, T, E, k, dgates, gates, idx, dlogits);
  return hipGetLastError();
}

}  // namespace moe
