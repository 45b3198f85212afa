// Row movement between token order and the packed per-expert buffers.
//
// Dispatch writes every routed token row straight into its expert's input buffer
// (rowwise dispatch: unite.ai, "Ai2 κυκλοφορεί το Olmo-Core 3…", section
// "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"; ettayeb.fr, "Olmo-core 3 ouvre
// l'entraînement des MoE…", section "Trois parallélismes, trois optimisations de
// routage"); combine gathers the expert outputs back per token, weighted by the gates.
// All four kernels are HBM-bound row copies: one wavefront per token, 16-byte accesses,
// consecutive lanes on consecutive 16-byte chunks of a row, float accumulation in a
// fixed order (j = 0..k-1), no atomics.
#include "common.h"
#include "route.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = kThreads / kWave;

// x_perm[slot_row[t, j]] = x[t]; row_src[slot_row[t, j]] = t
template <typename T>
__global__ void __launch_bounds__(kThreads) permute_kernel(int ntok, int d, int k, const T* __restrict__ x,
                                                           const int32_t* __restrict__ slot_row,
                                                           int32_t* __restrict__ row_src, T* __restrict__ x_perm) {
  const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= ntok) return;
  constexpr int V = 16 / sizeof(T);
  const int nchunk = d / V;
  const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * d);
  for (int c = lane; c < nchunk; c += kWave) {
    const uint4 v = src[c];
    for (int j = 0; j < k; j++) {
      const int r = slot_row[(int64_t)t * k + j];
      reinterpret_cast<uint4*>(x_perm + (int64_t)r * d)[c] = v;
    }
  }
  if (row_src && lane < k) row_src[slot_row[(int64_t)t * k + lane]] = t;
}

// Gathers (combine, un-permute) read k rows per token: a wave takes its token's slot rows
// and gates into lanes once (broadcast with shuffles), then issues the loads of U 16-byte
// chunks of all k rows before any arithmetic.  k <= 4 runs four chunks per lane and pass
// (a whole 2048-wide row per wave pass; cold at T = 8192, d = 2048, E = 128 that was 8-9%
// faster than two for combine and un-permute), k <= 8 two, larger k one row at a time.

template <typename T>
__device__ __forceinline__ void widen8(const uint4& q, float (&v)[8]);
template <>
__device__ __forceinline__ void widen8<bf16_t>(const uint4& q, float (&v)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// y[t] = y_add[t] + sum_j gates[t, j] * y_perm[slot_row[t, j]]   (y_add may be null).
// KG > 0 (bf16, k <= KG): U chunks per lane and pass, all k rows' loads issued first.
template <typename T, int KG, int U>
__global__ void __launch_bounds__(kThreads) combine_kernel(int ntok, int d, int k, const T* __restrict__ y_perm,
                                                           const float* __restrict__ gates,
                                                           const int32_t* __restrict__ slot_row,
                                                           const T* __restrict__ y_add, T* __restrict__ y) {
  const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= ntok) return;
  const int nchunk = d / 8;
  if constexpr (KG > 0) {
    const int my_r = lane < k ? slot_row[(int64_t)t * k + lane] : 0;
    const float my_g = lane < k ? gates[(int64_t)t * k + lane] : 0.f;
    for (int c0 = lane; c0 < nchunk; c0 += U * kWave) {
      uint4 q[U][KG + 1];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        q[u][KG] = make_uint4(0, 0, 0, 0);
        if (y_add && c < nchunk) q[u][KG] = *reinterpret_cast<const uint4*>(y_add + (int64_t)t * d + c * 8);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          const int r = __shfl(my_r, j, kWave);
          if (j < k && c < nchunk) q[u][j] = *reinterpret_cast<const uint4*>(y_perm + (int64_t)r * d + c * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        if (c >= nchunk) break;
        float acc[8];
        widen8<T>(q[u][KG], acc);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          if (j >= k) break;
          const float g = __shfl(my_g, j, kWave);
          float v[8];
          widen8<T>(q[u][j], v);
#pragma unroll
          for (int i = 0; i < 8; i++) acc[i] = fmaf(g, v[i], acc[i]);
        }
        store8<T>(y + (int64_t)t * d + c * 8, acc);
      }
    }
    return;
  }
  for (int c = lane; c < nchunk; c += kWave) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (y_add) load8<T>(y_add + (int64_t)t * d + c * 8, acc);
    for (int j = 0; j < k; j++) {
      const int r = slot_row[(int64_t)t * k + j];
      const float g = gates[(int64_t)t * k + j];
      float v[8];
      load8<T>(y_perm + (int64_t)r * d + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = fmaf(g, v[i], acc[i]);
    }
    store8<T>(y + (int64_t)t * d + c * 8, acc);
  }
}

// dy_perm[slot_row[t, j]] = gates[t, j] * dy[t];  dgates[t, j] = <dy[t], y_perm[slot_row[t, j]]>.
// KG > 0 (bf16, k <= KG): dy read once per chunk, U chunks per lane and pass with all k
// rows' loads issued first.  Each lane sums its chunks in ascending order whatever U is.
template <typename T, int KG, int U>
__global__ void __launch_bounds__(kThreads) combine_bwd_kernel(int ntok, int d, int k, const T* __restrict__ dy,
                                                               const T* __restrict__ y_perm,
                                                               const float* __restrict__ gates,
                                                               const int32_t* __restrict__ slot_row,
                                                               T* __restrict__ dy_perm, float* __restrict__ dgates) {
  const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= ntok) return;
  const int nchunk = d / 8;
  if constexpr (KG > 0) {
    const int my_r = lane < k ? slot_row[(int64_t)t * k + lane] : 0;
    const float my_g = lane < k ? gates[(int64_t)t * k + lane] : 0.f;
    float dot[KG];
#pragma unroll
    for (int j = 0; j < KG; j++) dot[j] = 0.f;
    for (int c0 = lane; c0 < nchunk; c0 += U * kWave) {
      uint4 q[U][KG + 1];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        if (c < nchunk) q[u][KG] = *reinterpret_cast<const uint4*>(dy + (int64_t)t * d + c * 8);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          const int r = __shfl(my_r, j, kWave);
          if (j < k && c < nchunk) q[u][j] = *reinterpret_cast<const uint4*>(y_perm + (int64_t)r * d + c * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        if (c >= nchunk) break;
        float du[8];
        widen8<T>(q[u][KG], du);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          if (j >= k) break;
          const int r = __shfl(my_r, j, kWave);
          const float g = __shfl(my_g, j, kWave);
          float v[8], o[8];
          widen8<T>(q[u][j], v);
#pragma unroll
          for (int i = 0; i < 8; i++) {
            dot[j] = fmaf(du[i], v[i], dot[j]);
            o[i] = g * du[i];
          }
          store8<T>(dy_perm + (int64_t)r * d + c * 8, o);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KG; j++) {
      if (j >= k) break;
      const float sj = wave_sum(dot[j]);
      if (lane == 0) dgates[(int64_t)t * k + j] = sj;
    }
    return;
  }
  for (int j = 0; j < k; j++) {
    const int r = slot_row[(int64_t)t * k + j];
    const float g = gates[(int64_t)t * k + j];
    float dot = 0.f;
    for (int c = lane; c < nchunk; c += kWave) {
      float u[8], v[8], o[8];
      load8<T>(dy + (int64_t)t * d + c * 8, u);
      load8<T>(y_perm + (int64_t)r * d + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        dot = fmaf(u[i], v[i], dot);
        o[i] = g * u[i];
      }
      store8<T>(dy_perm + (int64_t)r * d + c * 8, o);
    }
    dot = wave_sum(dot);
    if (lane == 0) dgates[(int64_t)t * k + j] = dot;
  }
}

// dgates[t, j] = <dy[t], y_perm[slot_row[t, j]]> alone (the routed gradient rows are
// written elsewhere).  Same per-lane order as combine_bwd_kernel (chunks ascending, the 8
// elements of a chunk in order, then a butterfly over the wave), so the two agree bit for
// bit; U chunks per lane and pass, the k rows' loads issued before any arithmetic.
template <int KG, int U>
__global__ void __launch_bounds__(kThreads) dgates_kernel(int ntok, int d, int k, const bf16_t* __restrict__ dy,
                                                          const bf16_t* __restrict__ y_perm,
                                                          const int32_t* __restrict__ slot_row,
                                                          float* __restrict__ dgates) {
  const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= ntok) return;
  const int nchunk = d / 8;
  if constexpr (KG == 0) {  // one row at a time
    for (int j = 0; j < k; j++) {
      const int r = slot_row[(int64_t)t * k + j];
      float dot = 0.f;
      for (int c = lane; c < nchunk; c += kWave) {
        float u[8], v[8];
        load8<bf16_t>(dy + (int64_t)t * d + c * 8, u);
        load8<bf16_t>(y_perm + (int64_t)r * d + c * 8, v);
#pragma unroll
        for (int i = 0; i < 8; i++) dot = fmaf(u[i], v[i], dot);
      }
      dot = wave_sum(dot);
      if (lane == 0) dgates[(int64_t)t * k + j] = dot;
    }
    return;
  } else {
    const int my_r = lane < k ? slot_row[(int64_t)t * k + lane] : 0;
    float dot[KG];
#pragma unroll
    for (int j = 0; j < KG; j++) dot[j] = 0.f;
    for (int c0 = lane; c0 < nchunk; c0 += U * kWave) {
      uint4 q[U][KG + 1];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        if (c < nchunk) q[u][KG] = *reinterpret_cast<const uint4*>(dy + (int64_t)t * d + c * 8);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          const int r = __shfl(my_r, j, kWave);
          if (j < k && c < nchunk) q[u][j] = *reinterpret_cast<const uint4*>(y_perm + (int64_t)r * d + c * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        if (c0 + u * kWave >= nchunk) break;
        float du[8];
        widen8<bf16_t>(q[u][KG], du);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          if (j >= k) break;
          float v[8];
          widen8<bf16_t>(q[u][j], v);
#pragma unroll
          for (int i = 0; i < 8; i++) dot[j] = fmaf(du[i], v[i], dot[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KG; j++) {
      if (j >= k) break;
      const float sm = wave_sum(dot[j]);
      if (lane == 0) dgates[(int64_t)t * k + j] = sm;
    }
  }
}

// row_src[slot_row[t, j]] = t
__global__ void row_src_kernel(int nslot, int k, const int32_t* __restrict__ slot_row, int32_t* __restrict__ row_src) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nslot) row_src[slot_row[i]] = i / k;
}

// dx[t] = dx_r[t] + dx_add[t] + sum_j dx_perm[slot_row[t, j]]   (dx_r, dx_add may be null).
// KG > 0 (bf16, k <= KG): U chunks per lane and pass, all loads issued first.
template <typename T, int KG, int U>
__global__ void __launch_bounds__(kThreads) unpermute_sum_kernel(int ntok, int d, int k, const T* __restrict__ dx_perm,
                                                                 const int32_t* __restrict__ slot_row,
                                                                 const T* __restrict__ dx_r,
                                                                 const T* __restrict__ dx_add, T* __restrict__ dx) {
  const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= ntok) return;
  const int nchunk = d / 8;
  if constexpr (KG > 0) {
    const int my_r = lane < k ? slot_row[(int64_t)t * k + lane] : 0;
    for (int c0 = lane; c0 < nchunk; c0 += U * kWave) {
      uint4 q[U][KG + 2];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        q[u][KG] = make_uint4(0, 0, 0, 0);
        q[u][KG + 1] = make_uint4(0, 0, 0, 0);
        if (dx_r && c < nchunk) q[u][KG] = *reinterpret_cast<const uint4*>(dx_r + (int64_t)t * d + c * 8);
        if (dx_add && c < nchunk) q[u][KG + 1] = *reinterpret_cast<const uint4*>(dx_add + (int64_t)t * d + c * 8);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          const int r = __shfl(my_r, j, kWave);
          if (j < k && c < nchunk) q[u][j] = *reinterpret_cast<const uint4*>(dx_perm + (int64_t)r * d + c * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        if (c >= nchunk) break;
        float acc[8], w[8];
        widen8<T>(q[u][KG], acc);
        widen8<T>(q[u][KG + 1], w);
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] += w[i];
#pragma unroll
        for (int j = 0; j < KG; j++) {
          if (j >= k) break;
          float v[8];
          widen8<T>(q[u][j], v);
#pragma unroll
          for (int i = 0; i < 8; i++) acc[i] += v[i];
        }
        store8<T>(dx + (int64_t)t * d + c * 8, acc);
      }
    }
    return;
  }
  for (int c = lane; c < nchunk; c += kWave) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (dx_r) load8<T>(dx_r + (int64_t)t * d + c * 8, acc);
    if (dx_add) {
      float w[8];
      load8<T>(dx_add + (int64_t)t * d + c * 8, w);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += w[i];
    }
    for (int j = 0; j < k; j++) {
      const int r = slot_row[(int64_t)t * k + j];
      float v[8];
      load8<T>(dx_perm + (int64_t)r * d + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += v[i];
    }
    store8<T>(dx + (int64_t)t * d + c * 8, acc);
  }
}

// dx[t] = dx_add[t] + sum_j (dx_perm[slot_row[t, j]] + dL[t, e_j] Wr[e_j]), e_j = topk_idx[t, j]:
// the un-permute with the router's input gradient dx_r = dL Wr folded in.  The gates are a
// softmax over the token's k chosen scores, so dL is zero outside those k experts and
// dx_r[t] has k terms, each a row of Wr (E rows of d, which stay in L2).  Float accumulation
// in the order dx_add, then per j the routed row and the fma of its router term; one
// rounding to the output type.  Expert ids are clamped into [0, E) before any Wr access.
// KG > 0 (bf16, k <= KG): U chunks per lane and pass, all 2k + 1 loads issued first.
template <typename T, int KG, int U>
__global__ void __launch_bounds__(kThreads) unpermute_router_kernel(int ntok, int d, int k, int E,
                                                                    const T* __restrict__ dx_perm,
                                                                    const int32_t* __restrict__ slot_row,
                                                                    const int32_t* __restrict__ topk_idx,
                                                                    const float* __restrict__ dL,
                                                                    const T* __restrict__ Wr,
                                                                    const T* __restrict__ dx_add, T* __restrict__ dx) {
  const int t = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= ntok) return;
  const int nchunk = d / 8;
  auto expert = [&](int j) {
    const int e = topk_idx[(int64_t)t * k + j];
    return e < 0 ? 0 : (e >= E ? E - 1 : e);
  };
  if constexpr (KG > 0) {
    const int my_r = lane < k ? slot_row[(int64_t)t * k + lane] : 0;
    const int my_e = lane < k ? expert(lane) : 0;
    const float my_g = lane < k ? dL[(int64_t)t * E + my_e] : 0.f;
    for (int c0 = lane; c0 < nchunk; c0 += U * kWave) {
      uint4 q[U][2 * KG + 1];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        q[u][2 * KG] = make_uint4(0, 0, 0, 0);
        if (dx_add && c < nchunk) q[u][2 * KG] = *reinterpret_cast<const uint4*>(dx_add + (int64_t)t * d + c * 8);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          const int r = __shfl(my_r, j, kWave), e = __shfl(my_e, j, kWave);
          if (j < k && c < nchunk) {
            q[u][j] = *reinterpret_cast<const uint4*>(dx_perm + (int64_t)r * d + c * 8);
            q[u][KG + j] = *reinterpret_cast<const uint4*>(Wr + (int64_t)e * d + c * 8);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * kWave;
        if (c >= nchunk) break;
        float acc[8];
        widen8<T>(q[u][2 * KG], acc);
#pragma unroll
        for (int j = 0; j < KG; j++) {
          if (j >= k) break;
          const float g = __shfl(my_g, j, kWave);
          float v[8], w[8];
          widen8<T>(q[u][j], v);
          widen8<T>(q[u][KG + j], w);
#pragma unroll
          for (int i = 0; i < 8; i++) acc[i] = fmaf(g, w[i], acc[i] + v[i]);
        }
        store8<T>(dx + (int64_t)t * d + c * 8, acc);
      }
    }
    return;
  }
  for (int c = lane; c < nchunk; c += kWave) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (dx_add) load8<T>(dx_add + (int64_t)t * d + c * 8, acc);
    for (int j = 0; j < k; j++) {
      const int r = slot_row[(int64_t)t * k + j];
      const int e = expert(j);
      const float g = dL[(int64_t)t * E + e];
      float v[8], w[8];
      load8<T>(dx_perm + (int64_t)r * d + c * 8, v);
      load8<T>(Wr + (int64_t)e * d + c * 8, w);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = fmaf(g, w[i], acc[i] + v[i]);
    }
    store8<T>(dx + (int64_t)t * d + c * 8, acc);
  }
}

inline dim3 tok_grid(int T) { return dim3((unsigned)((T + kTokPerBlock - 1) / kTokPerBlock)); }

}  // namespace

hipError_t permute_rows(int eb, int T, int d, int k, const void* x, const int32_t* slot_row, int32_t* row_src,
                        void* x_perm, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (eb == 2)
    hipLaunchKernelGGL(permute_kernel<bf16_t>, tok_grid(T), dim3(kThreads), 0, st, T, d, k, (const bf16_t*)x, slot_row,
                       row_src, (bf16_t*)x_perm);
  else
    hipLaunchKernelGGL(permute_kernel<float>, tok_grid(T), dim3(kThreads), 0, st, T, d, k, (const float*)x, slot_row,
                       row_src, (float*)x_perm);
  return hipGetLastError();
}

// bf16 gather kernels by the token's expert count: <KG, U> = <4, 4> for k <= 4, <8, 2> for
// k <= 8, one row at a time beyond.  fp32 rows always take the row-at-a-time loop.
hipError_t combine_rows(int eb, int T, int d, int k, const void* y_perm, const float* gates, const int32_t* slot_row,
                        const void* y_add, void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (eb == 2) {
    if (k <= 4)
      hipLaunchKernelGGL((combine_kernel<bf16_t, 4, 4>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)y_perm, gates, slot_row, (const bf16_t*)y_add, (bf16_t*)y);
    else if (k <= 8)
      hipLaunchKernelGGL((combine_kernel<bf16_t, 8, 2>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)y_perm, gates, slot_row, (const bf16_t*)y_add, (bf16_t*)y);
    else
      hipLaunchKernelGGL((combine_kernel<bf16_t, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)y_perm, gates, slot_row, (const bf16_t*)y_add, (bf16_t*)y);
  } else {
    hipLaunchKernelGGL((combine_kernel<float, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k, (const float*)y_perm,
                       gates, slot_row, (const float*)y_add, (float*)y);
  }
  return hipGetLastError();
}

hipError_t combine_rows_bwd(int eb, int T, int d, int k, const void* dy, const void* y_perm, const float* gates,
                            const int32_t* slot_row, void* dy_perm, float* dgates, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (eb == 2) {
    if (k <= 4)
      hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, 4, 4>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)dy, (const bf16_t*)y_perm, gates, slot_row, (bf16_t*)dy_perm, dgates);
    else if (k <= 8)
      hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, 8, 2>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)dy, (const bf16_t*)y_perm, gates, slot_row, (bf16_t*)dy_perm, dgates);
    else
      hipLaunchKernelGGL((combine_bwd_kernel<bf16_t, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)dy, (const bf16_t*)y_perm, gates, slot_row, (bf16_t*)dy_perm, dgates);
  } else {
    hipLaunchKernelGGL((combine_bwd_kernel<float, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                       (const float*)dy, (const float*)y_perm, gates, slot_row, (float*)dy_perm, dgates);
  }
  return hipGetLastError();
}

hipError_t dgates_rows(int T, int d, int k, const bf16_t* dy, const bf16_t* y_perm, const int32_t* slot_row,
                       float* dgates, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (k <= 4)
    hipLaunchKernelGGL((dgates_kernel<4, 4>), tok_grid(T), dim3(kThreads), 0, st, T, d, k, dy, y_perm, slot_row, dgates);
  else if (k <= 8)
    hipLaunchKernelGGL((dgates_kernel<8, 2>), tok_grid(T), dim3(kThreads), 0, st, T, d, k, dy, y_perm, slot_row, dgates);
  else
    hipLaunchKernelGGL((dgates_kernel<0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k, dy, y_perm, slot_row, dgates);
  return hipGetLastError();
}

hipError_t row_src_rows(int T, int k, const int32_t* slot_row, int32_t* row_src, hipStream_t st) {
  const int64_t n = (int64_t)T * k;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(row_src_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (int)n, k, slot_row, row_src);
  return hipGetLastError();
}

hipError_t unpermute_sum_rows(int eb, int T, int d, int k, const void* dx_perm, const int32_t* slot_row,
                              const void* dx_r, const void* dx_add, void* dx, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (eb == 2) {
    if (k <= 4)
      hipLaunchKernelGGL((unpermute_sum_kernel<bf16_t, 4, 4>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)dx_perm, slot_row, (const bf16_t*)dx_r, (const bf16_t*)dx_add, (bf16_t*)dx);
    else if (k <= 8)
      hipLaunchKernelGGL((unpermute_sum_kernel<bf16_t, 8, 2>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)dx_perm, slot_row, (const bf16_t*)dx_r, (const bf16_t*)dx_add, (bf16_t*)dx);
    else
      hipLaunchKernelGGL((unpermute_sum_kernel<bf16_t, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                         (const bf16_t*)dx_perm, slot_row, (const bf16_t*)dx_r, (const bf16_t*)dx_add, (bf16_t*)dx);
  } else {
    hipLaunchKernelGGL((unpermute_sum_kernel<float, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k,
                       (const float*)dx_perm, slot_row, (const float*)dx_r, (const float*)dx_add, (float*)dx);
  }
  return hipGetLastError();
}

hipError_t unpermute_router_rows(int eb, int T, int d, int k, int E, const void* dx_perm, const int32_t* slot_row,
                                 const int32_t* topk_idx, const float* dL, const void* Wr, const void* dx_add,
                                 void* dx, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (eb == 2) {
    if (k <= 4)
      hipLaunchKernelGGL((unpermute_router_kernel<bf16_t, 4, 2>), tok_grid(T), dim3(kThreads), 0, st, T, d, k, E,
                         (const bf16_t*)dx_perm, slot_row, topk_idx, dL, (const bf16_t*)Wr, (const bf16_t*)dx_add,
                         (bf16_t*)dx);
    else
      hipLaunchKernelGGL((unpermute_router_kernel<bf16_t, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k, E,
                         (const bf16_t*)dx_perm, slot_row, topk_idx, dL, (const bf16_t*)Wr, (const bf16_t*)dx_add,
                         (bf16_t*)dx);
  } else {
    hipLaunchKernelGGL((unpermute_router_kernel<float, 0, 1>), tok_grid(T), dim3(kThreads), 0, st, T, d, k, E,
                       (const float*)dx_perm, slot_row, topk_idx, dL, (const float*)Wr, (const float*)dx_add,
                       (float*)dx);
  }
  return hipGetLastError();
}

}  // namespace moe
