// MXFP8 block quantisation on the device: bf16 -> E4M3 codes + one E8M0 scale per 32
// elements.  MXFP8 is the reduced-precision format the pages report for the expert FFN
// compute and expert data movement (unite.ai, "Ai2 κυκλοφορεί το Olmo-Core 3…",
// section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"; ettayeb.fr, "Olmo-core 3
// ouvre l'entraînement des MoE…", section "Trois parallélismes, trois optimisations de
// routage").
//
// Scale: the smallest 2^s with amax * 2^-s <= 448 (E4M3's largest finite value),
// s clamped to [-127, 127]; blocks whose amax is zero or an fp32 subnormal get -127.
// Elements: round-to-nearest-even onto the E4M3 grid, done with integer arithmetic on
// the fp32 bit pattern (exact: the scaled value v * 2^-s is exact in fp32).
#include "common.h"
#include "mx.h"

namespace moe {

__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int eb = (int)((u >> 23) & 0xff);
  if (eb == 0) return -127;
  int s = eb - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);  // mantissa above 1.75 -> next power
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// |v| <= 448 finite -> E4M3 code, round to nearest even
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t au = __float_as_uint(a);
    int e = (int)((au >> 23) & 0xff) - 127;  // -6 .. 8
    const uint32_t m23 = au & 0x7fffffu;
    uint32_t m = (m23 + 0x7ffffu + ((m23 >> 20) & 1u)) >> 20;  // RNE to 3 bits: 0..8
    if (m == 8) { m = 0; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | m;
    if (code > 0x7eu) code = 0x7eu;          // guard: never reached for |v| <= 448
  }
  return sign | code;
}

__device__ __forceinline__ float exp2i(int s) { return __uint_as_float((uint32_t)(s + 127) << 23); }  // 2^s, s in [-126,127]

namespace {

// one thread per 32-element block of a row
__global__ void mx_rows_kernel(int rows, int cols, const bf16_t* __restrict__ src, uint8_t* __restrict__ q,
                               uint8_t* __restrict__ scales) {
  const int nb = cols / kMxBlock;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= (int64_t)rows * nb) return;
  const bf16_t* p = src + b * kMxBlock;
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    float t[8];
    load8<bf16_t>(p + 8 * i, t);
#pragma unroll
    for (int j = 0; j < 8; j++) v[8 * i + j] = t[j];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
  const int s = mx_scale_exp(amax);
  // 2^-s as a product of two normal powers so s = -127 (2^127) and s = 127 stay exact
  const float r1 = exp2i(-s / 2), r2 = exp2i(-s - (-s / 2));
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    w[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) w[i] |= e4m3_rne(v[4 * i + j] * r1 * r2) << (8 * j);
  }
  uint4* o = reinterpret_cast<uint4*>(q + b * kMxBlock);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[b] = (uint8_t)(s + 127);
}

// Transposed, segment-restarting quantisation: thread (block, column).  Segment e's
// rows land in columns [P_e, P_e + roundup(n_e, kMxSegPad)) of the [cols, rows_pad]
// output; padding gets zero codes and zero-block scales.
__global__ void mx_cols_seg_kernel(int rows, int cols, int rows_pad, const int32_t* __restrict__ seg, int nseg,
                                   const bf16_t* __restrict__ src, uint8_t* __restrict__ q,
                                   uint8_t* __restrict__ scales) {
  __shared__ int s_pstart[kMaxExperts + 1];
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < nseg; e++) {
      s_pstart[e] = acc;
      const int n = seg[e + 1] - seg[e];
      acc += (n + kMxSegPad - 1) / kMxSegPad * kMxSegPad;
    }
    s_pstart[nseg] = acc;
  }
  __syncthreads();
  const int c = blockIdx.x * blockDim.x + threadIdx.x;  // column
  const int pb = blockIdx.y;                             // padded 32-row block
  if (c >= cols) return;
  const int prow = pb * kMxBlock;
  if (prow >= s_pstart[nseg]) return;
  int lo = 0, hi = nseg;  // segment with s_pstart[e] <= prow < s_pstart[e+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pstart[mid] <= prow) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int r0 = seg[e] + (prow - s_pstart[e]);
  const int r1 = seg[e + 1];
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const int r = r0 + i;
    v[i] = r < r1 ? bf2f(src[(int64_t)r * cols + c]) : 0.f;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int s = mx_scale_exp(amax);
  const float f1 = exp2i(-s / 2), f2 = exp2i(-s - (-s / 2));
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    w[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) w[i] |= e4m3_rne(v[4 * i + j] * f1 * f2) << (8 * j);
  }
  uint4* o = reinterpret_cast<uint4*>(q + (int64_t)c * rows_pad + prow);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[(int64_t)c * (rows_pad / kMxBlock) + pb] = (uint8_t)(s + 127);
}

}  // namespace

hipError_t mx_quantize_rows(int rows, int cols, const bf16_t* src, uint8_t* q, uint8_t* scales, hipStream_t st) {
  const int64_t n = (int64_t)rows * (cols / kMxBlock);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, rows, cols, src, q, scales);
  return hipGetLastError();
}

hipError_t mx_quantize_cols_seg(int rows, int cols, const int32_t* seg_offsets, int nseg, const bf16_t* src,
                                uint8_t* q, uint8_t* scales, hipStream_t st) {
  const int rows_pad = rows + kMxSegPad * nseg;
  dim3 grid((unsigned)((cols + 255) / 256), (unsigned)(rows_pad / kMxBlock));
  hipLaunchKernelGGL(mx_cols_seg_kernel, grid, dim3(256), 0, st, rows, cols, rows_pad, seg_offsets, nseg, src, q,
                     scales);
  return hipGetLastError();
}

size_t mx_workspace_bytes(int R, int d, int f, int E) { return 0; }

hipError_t gemm1_fwd_mx(const GemmShape&, const int*, const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*, bf16_t*,
                        void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t gemm2_fwd_mx(const GemmShape&, const int*, const bf16_t*, const bf16_t*, bf16_t*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t dgrad2_mx(const GemmShape&, const int*, const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*, void*,
                     hipStream_t) { return hipErrorNotSupported; }
hipError_t wgrad2_mx(const GemmShape&, const int*, const bf16_t*, const bf16_t*, bf16_t*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t dgrad1_mx(const GemmShape&, const int*, const bf16_t*, const bf16_t*, const bf16_t*, bf16_t*, void*,
                     hipStream_t) { return hipErrorNotSupported; }
hipError_t wgrad1_mx(const GemmShape&, const int*, const bf16_t*, const bf16_t*, bf16_t*, bf16_t*, void*,
                     hipStream_t) { return hipErrorNotSupported; }

}  // namespace moe
