// Float32 expert and router GEMMs: plain FMA kernels, one output element per thread.
// They serve the fp32 workload (small shapes, checked to 1e-4 normwise); the bf16 and
// MXFP8 paths run on the matrix cores.  Same grouping rules as the bf16 grouped GEMM:
// rows [offsets[e], offsets[e+1]) of the packed buffers belong to expert e.
#include "common.h"
#include "gemm.h"

namespace moe {
namespace {

__device__ __forceinline__ int find_segment(const int* offsets, int E, int r) {
  int lo = 0, hi = E;  // largest e with offsets[e] <= r
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// a = X W1_e^T, b = X W3_e^T, h = silu(a) b; one thread per (row, hidden column)
__global__ void gemm1_f32_kernel(GemmShape s, const int* off, const float* X, const float* W1, const float* W3,
                                 float* ab, float* h) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)s.R * s.f) return;
  const int r = (int)(idx / s.f), c = (int)(idx % s.f);
  const int e = find_segment(off, s.E, r);
  const float* x = X + (int64_t)r * s.d;
  const float* w1 = W1 + ((int64_t)e * s.f + c) * s.d;
  const float* w3 = W3 + ((int64_t)e * s.f + c) * s.d;
  float a = 0.f, b = 0.f;
  for (int k = 0; k < s.d; k++) { a = fmaf(x[k], w1[k], a); b = fmaf(x[k], w3[k], b); }
  ab[(int64_t)r * 2 * s.f + c] = a;
  ab[(int64_t)r * 2 * s.f + s.f + c] = b;
  h[(int64_t)r * s.f + c] = a * sigmoidf_(a) * b;
}

// y = h W2_e^T
__global__ void gemm2_f32_kernel(GemmShape s, const int* off, const float* H, const float* W2, float* Y) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)s.R * s.d) return;
  const int r = (int)(idx / s.d), n = (int)(idx % s.d);
  const int e = find_segment(off, s.E, r);
  const float* hr = H + (int64_t)r * s.f;
  const float* w = W2 + ((int64_t)e * s.d + n) * s.f;
  float acc = 0.f;
  for (int k = 0; k < s.f; k++) acc = fmaf(hr[k], w[k], acc);
  Y[(int64_t)r * s.d + n] = acc;
}

// dh = dy W2_e, then da, db from the saved a, b
__global__ void dgrad2_f32_kernel(GemmShape s, const int* off, const float* dY, const float* W2, const float* ab,
                                  float* dab) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)s.R * s.f) return;
  const int r = (int)(idx / s.f), c = (int)(idx % s.f);
  const int e = find_segment(off, s.E, r);
  const float* dy = dY + (int64_t)r * s.d;
  const float* w = W2 + (int64_t)e * s.d * s.f + c;
  float dh = 0.f;
  for (int k = 0; k < s.d; k++) dh = fmaf(dy[k], w[(int64_t)k * s.f], dh);
  const float a = ab[(int64_t)r * 2 * s.f + c], b = ab[(int64_t)r * 2 * s.f + s.f + c];
  const float sg = sigmoidf_(a);
  dab[(int64_t)r * 2 * s.f + c] = dh * b * sg * (1.f + a * (1.f - sg));
  dab[(int64_t)r * 2 * s.f + s.f + c] = dh * a * sg;
}

// dW2_e[m, n] = sum_r dy[r, m] h[r, n]
__global__ void wgrad2_f32_kernel(GemmShape s, const int* off, const float* H, const float* dY, float* dW2) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)s.E * s.d * s.f) return;
  const int e = (int)(idx / ((int64_t)s.d * s.f));
  const int m = (int)((idx / s.f) % s.d), n = (int)(idx % s.f);
  float acc = 0.f;
  for (int r = off[e]; r < off[e + 1]; r++) acc = fmaf(dY[(int64_t)r * s.d + m], H[(int64_t)r * s.f + n], acc);
  dW2[idx] = acc;
}

// dx = da W1_e + db W3_e
__global__ void dgrad1_f32_kernel(GemmShape s, const int* off, const float* dab, const float* W1, const float* W3,
                                  float* dX) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)s.R * s.d) return;
  const int r = (int)(idx / s.d), n = (int)(idx % s.d);
  const int e = find_segment(off, s.E, r);
  const float* g = dab + (int64_t)r * 2 * s.f;
  const float* w1 = W1 + (int64_t)e * s.f * s.d + n;
  const float* w3 = W3 + (int64_t)e * s.f * s.d + n;
  float acc = 0.f;
  for (int k = 0; k < s.f; k++) acc = fmaf(g[k], w1[(int64_t)k * s.d], acc);
  for (int k = 0; k < s.f; k++) acc = fmaf(g[s.f + k], w3[(int64_t)k * s.d], acc);
  dX[(int64_t)r * s.d + n] = acc;
}

// dW1_e[m, n] = sum_r da[r, m] x[r, n]; dW3 likewise with db
__global__ void wgrad1_f32_kernel(GemmShape s, const int* off, const float* X, const float* dab, float* dW1,
                                  float* dW3) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)s.E * 2 * s.f * s.d) return;
  const int e = (int)(idx / ((int64_t)2 * s.f * s.d));
  const int m = (int)((idx / s.d) % (2 * s.f)), n = (int)(idx % s.d);
  float acc = 0.f;
  for (int r = off[e]; r < off[e + 1]; r++) acc = fmaf(dab[(int64_t)r * 2 * s.f + m], X[(int64_t)r * s.d + n], acc);
  float* W = m < s.f ? dW1 + ((int64_t)e * s.f + m) * s.d : dW3 + ((int64_t)e * s.f + (m - s.f)) * s.d;
  W[n] = acc;
}

__global__ void router_fwd_f32_kernel(int T, int d, int E, const float* X, const float* Wr, const float* bias,
                                      float* L) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * E) return;
  const int t = (int)(idx / E), e = (int)(idx % E);
  float acc = 0.f;
  for (int k = 0; k < d; k++) acc = fmaf(X[(int64_t)t * d + k], Wr[(int64_t)e * d + k], acc);
  L[idx] = acc + (bias ? bias[e] : 0.f);
}

__global__ void router_dx_f32_kernel(int T, int d, int E, const float* dL, const float* Wr, float* dX) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * d) return;
  const int t = (int)(idx / d), n = (int)(idx % d);
  float acc = 0.f;
  for (int e = 0; e < E; e++) acc = fmaf(dL[(int64_t)t * E + e], Wr[(int64_t)e * d + n], acc);
  dX[idx] = acc;
}

__global__ void router_dw_f32_kernel(int T, int d, int E, const float* dL, const float* X, float* dW) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)E * d) return;
  const int e = (int)(idx / d), n = (int)(idx % d);
  float acc = 0.f;
  for (int t = 0; t < T; t++) acc = fmaf(dL[(int64_t)t * E + e], X[(int64_t)t * d + n], acc);
  dW[idx] = acc;
}

inline dim3 grid_for(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

}  // namespace

#define MOE_LAUNCH_F32(kernel, count, ...)                                  \
  do {                                                                       \
    if ((count) == 0) return hipSuccess;                                    \
    hipLaunchKernelGGL(kernel, grid_for(count), dim3(256), 0, st, __VA_ARGS__); \
    return hipGetLastError();                                                \
  } while (0)

hipError_t gemm1_fwd_f32(const GemmShape& s, const int* o, const float* X, const float* W1, const float* W3,
                         float* ab, float* h, hipStream_t st) {
  MOE_LAUNCH_F32(gemm1_f32_kernel, (int64_t)s.R * s.f, s, o, X, W1, W3, ab, h);
}
hipError_t gemm2_fwd_f32(const GemmShape& s, const int* o, const float* H, const float* W2, float* Y,
                         hipStream_t st) {
  MOE_LAUNCH_F32(gemm2_f32_kernel, (int64_t)s.R * s.d, s, o, H, W2, Y);
}
hipError_t dgrad2_f32(const GemmShape& s, const int* o, const float* dY, const float* W2, const float* ab,
                      float* dab, hipStream_t st) {
  MOE_LAUNCH_F32(dgrad2_f32_kernel, (int64_t)s.R * s.f, s, o, dY, W2, ab, dab);
}
hipError_t wgrad2_f32(const GemmShape& s, const int* o, const float* H, const float* dY, float* dW2,
                      hipStream_t st) {
  MOE_LAUNCH_F32(wgrad2_f32_kernel, (int64_t)s.E * s.d * s.f, s, o, H, dY, dW2);
}
hipError_t dgrad1_f32(const GemmShape& s, const int* o, const float* dab, const float* W1, const float* W3,
                      float* dX, hipStream_t st) {
  MOE_LAUNCH_F32(dgrad1_f32_kernel, (int64_t)s.R * s.d, s, o, dab, W1, W3, dX);
}
hipError_t wgrad1_f32(const GemmShape& s, const int* o, const float* X, const float* dab, float* dW1,
                      float* dW3, hipStream_t st) {
  MOE_LAUNCH_F32(wgrad1_f32_kernel, (int64_t)s.E * 2 * s.f * s.d, s, o, X, dab, dW1, dW3);
}
hipError_t router_fwd_f32(int T, int d, int E, const float* X, const float* Wr, const float* bias, float* L,
                          hipStream_t st) {
  MOE_LAUNCH_F32(router_fwd_f32_kernel, (int64_t)T * E, T, d, E, X, Wr, bias, L);
}
hipError_t router_dx_f32(int T, int d, int E, const float* dL, const float* Wr, float* dX, hipStream_t st) {
  MOE_LAUNCH_F32(router_dx_f32_kernel, (int64_t)T * d, T, d, E, dL, Wr, dX);
}
hipError_t router_dw_f32(int T, int d, int E, const float* dL, const float* X, float* dW, hipStream_t st) {
  MOE_LAUNCH_F32(router_dw_f32_kernel, (int64_t)E * d, T, d, E, dL, X, dW);
}

}  // namespace moe
