// Grouped GEMM on gfx950 matrix cores (bf16 operands, fp32 accumulation).
//
// One kernel template serves every expert GEMM of the layer (and the router GEMMs):
// a grouped GEMM over many small expert computations whose group boundaries live only
// on the device (unite.ai, "Ai2 κυκλοφορεί το Olmo-Core 3…", section "Παραλληλισμός,
// Ακρίβεια και Τεχνικές Μνήμης": grouped GEMM, GPU-resident routing, device-scheduled
// grouped matmuls).  The grid is persistent and sized from host-known shapes only; each
// workgroup rebuilds the tile map from `offsets` in LDS, so the host never learns the
// per-expert counts.
//
//   GROUP_M  rows of A and C are grouped by expert (forward and data-gradient GEMMs):
//            C[r, n] = sum_k A[r, k] * B_e[k, n] for r in [offsets[e], offsets[e+1]).
//   GROUP_K  the reduction is grouped by expert (weight-gradient GEMMs):
//            C_e[m, n] = sum_{r in [offsets[e], offsets[e+1])} A[r, m] * B[r, n].
//
// An operand whose reduction axis is contiguous in memory ("K-contiguous") is kept
// [mn][k] in LDS and read with 16-byte ds_read_b128; an operand contiguous along M or N
// is kept [k][mn] as loaded and read with the gfx950 transpose read ds_read_b64_tr_b16,
// so no operand is ever transposed in HBM.  MFMA: v_mfma_f32_32x32x16_bf16 (lane l holds
// row l%32, k = 8*(l/32)..+7 of A; column l%32 of B; accumulator row 8*(i/4)+4*(l/32)+i%4).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "common.h"
#include "gemm.h"
#include "tilemap.h"
#include "epilogue.h"

namespace moe {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------------------------------
// Problem descriptions (operand addressing + epilogue) for each GEMM of the layer.
// seg(e): start row of group e -- from the routing offsets, or uniform splits of
// seg_len rows (single-group GEMMs and split reductions).
// ---------------------------------------------------------------------------------------
struct ProbBase {
  static constexpr bool MXQ = false;  // no MXFP8 copy of the output
  static constexpr bool N_MAJOR = true;  // Group::M tile order within an expert
  static constexpr bool STORE16 = false;  // bf16 output rows through out_row (Epi::Store)
  int M = 0, N = 0, K = 0, E = 1;
  const int* offsets = nullptr;
  int seg_len = 0, seg_total = 0;
  __device__ int seg(int e) const {
    if (offsets) return offsets[e];
    const int64_t v = (int64_t)e * seg_len;
    return v < seg_total ? (int)v : seg_total;
  }
  // B rows that change tensor at k = k_split() (the pipelined kernel restarts its address
  // streams there)
  static constexpr bool K_SPLIT = false;
  __device__ int k_split() const { return 0; }
};

// Forward GEMM1 with the SwiGLU epilogue: [a | b] = X_e [W1_e | W3_e]^T, the B tile's
// 32-column blocks alternate W1 / W3 rows so each wave holds a and b of the same column.
// Q: h is also written as MXFP8 row blocks (codes hq [R][f], scales hs [R][f/32]), the
// operand of an MXFP8 GEMM2.
template <bool Q>
struct ProbGemm1T : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = true;
  static constexpr Epi EPI = Epi::SwiGLU;
  static constexpr bool MXQ = Q;
  int f = 0;
  const bf16_t* X = nullptr; const bf16_t* W1 = nullptr; const bf16_t* W3 = nullptr;
  bf16_t* ab = nullptr; bf16_t* h = nullptr;
  uint8_t* hq = nullptr; uint8_t* hs = nullptr;
  __device__ const bf16_t* a_row(int, int m) const { return X + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int n) const {
    const int blk = n >> 5, col = (blk >> 1) * 32 + (n & 31);
    const bf16_t* W = (blk & 1) ? W3 : W1;
    return W + ((int64_t)e * f + col) * K;
  }
  __device__ void swiglu4(const float (&a)[4], const float (&b)[4], float (&hv)[4]) const {
#pragma unroll
    for (int c = 0; c < 4; c++) hv[c] = a[c] * sigmoidf_(a[c]) * b[c];
  }
  __device__ void epilogue_swiglu4(int m, int hcol, const float (&a)[4], const float (&b)[4]) const {
    bf16_t* abr = ab + (int64_t)m * 2 * f;
    store_bf16x4(abr + hcol, a);
    store_bf16x4(abr + f + hcol, b);
    float hv[4];
    swiglu4(a, b, hv);
    store_bf16x4(h + (int64_t)m * f + hcol, hv);
  }
  static constexpr bool STORE16 = true;
  // 8 columns hcol .. hcol+7 of row m, packed bf16: a, b into ab, h into h
  __device__ void store_swiglu16(int m, int hcol, const uint4& a, const uint4& b, const uint4& hv) const {
    bf16_t* abr = ab + (int64_t)m * 2 * f;
    *reinterpret_cast<uint4*>(abr + hcol) = a;
    *reinterpret_cast<uint4*>(abr + f + hcol) = b;
    *reinterpret_cast<uint4*>(h + (int64_t)m * f + hcol) = hv;
  }
  __device__ void store_swiglu16_q(int m, int hcol, const uint4& hv, bool valid, bool first) const {
    mx_block_store8(hv, valid, hq + (int64_t)m * f + hcol, hs + (int64_t)m * (f / 32) + hcol / 32, first);
  }
  __device__ void epilogue_swiglu4_q(int m, int hcol, const float (&a)[4], const float (&b)[4], bool valid,
                                     int quad) const {
    float hv[4];
    swiglu4(a, b, hv);
    if (valid) {
      bf16_t* abr = ab + (int64_t)m * 2 * f;
      store_bf16x4(abr + hcol, a);
      store_bf16x4(abr + f + hcol, b);
      store_bf16x4(h + (int64_t)m * f + hcol, hv);
    }
    mx_block_store4(hv, valid, hq + (int64_t)m * f + hcol, hs + (int64_t)m * (f / 32) + hcol / 32, quad);
  }
};
using ProbGemm1 = ProbGemm1T<false>;

// y_perm = h W2_e^T
struct ProbGemm2 : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = true;
  static constexpr Epi EPI = Epi::Store;
  const bf16_t* Hm = nullptr; const bf16_t* W2 = nullptr;
  bf16_t* Y = nullptr;
  __device__ const bf16_t* a_row(int, int m) const { return Hm + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int n) const { return W2 + ((int64_t)e * N + n) * K; }
  static constexpr bool STORE16 = true;
  __device__ bf16_t* out_row(int, int m) const { return Y + (int64_t)m * N; }
  __device__ void epilogue4(int, int m, int n, const float (&v)[4]) const { store_bf16x4(Y + (int64_t)m * N + n, v); }
};

// dh = dy_e W2_e (B = W2_e read [k=d][n=f]) with the SwiGLU-gradient epilogue.  Q: [da | db]
// is also written as MXFP8 row blocks (codes dq [R][2f], scales ds [R][2f/32]), the operand
// of an MXFP8 dgrad1.
template <bool Q>
struct ProbDgrad2T : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = false;
  static constexpr Epi EPI = Epi::DSwiGLU;
  static constexpr bool MXQ = Q;
  // M-tile major: N-tile major measured 6% slower here at E = 128, T = 8192 (its epilogue
  // reads the saved a, b of the tile's rows)
  static constexpr bool N_MAJOR = false;
  const bf16_t* dY = nullptr; const bf16_t* W2 = nullptr; const bf16_t* ab = nullptr;
  bf16_t* dab = nullptr;
  uint8_t* dq = nullptr; uint8_t* ds = nullptr;
  __device__ const bf16_t* a_row(int, int m) const { return dY + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int k) const { return W2 + ((int64_t)e * K + k) * N; }
  __device__ AbPair prefetch4(int m, int n) const { return load_ab4(ab, N, m, n); }
  __device__ void epilogue4_pre(int, int m, int n, const float (&dh)[4], const AbPair& pr) const {
    dswiglu_store4(dab, N, m, n, dh, pr);
  }
  static constexpr bool STORE16 = true;
  // 8 columns n .. n+7 of row m, packed bf16: da into dab[m][n], db into dab[m][N + n]
  __device__ void store_dswiglu16(int m, int n, const uint4& da, const uint4& db) const {
    bf16_t* o = dab + (int64_t)m * 2 * N;
    *reinterpret_cast<uint4*>(o + n) = da;
    *reinterpret_cast<uint4*>(o + N + n) = db;
  }
  __device__ void store_dswiglu16_q(int m, int n, const uint4& da, const uint4& db, bool valid, bool first) const {
    uint8_t* q = dq + (int64_t)m * 2 * N;
    uint8_t* sc = ds + (int64_t)m * (2 * N / 32);
    mx_block_store8(da, valid, q + n, sc + n / 32, first);
    mx_block_store8(db, valid, q + N + n, sc + (N + n) / 32, first);
  }
  __device__ void epilogue4_pre_q(int, int m, int n, const float (&dh)[4], const AbPair& pr, bool valid,
                                  int quad) const {
    float da[4], db[4];
    dswiglu4(dh, pr, da, db);
    if (valid) {
      bf16_t* o = dab + (int64_t)m * 2 * N;
      store_bf16x4(o + n, da);
      store_bf16x4(o + N + n, db);
    }
    uint8_t* q = dq + (int64_t)m * 2 * N;
    uint8_t* sc = ds + (int64_t)m * (2 * N / 32);
    mx_block_store4(da, valid, q + n, sc + n / 32, quad);
    mx_block_store4(db, valid, q + N + n, sc + (N + n) / 32, quad);
  }
};
using ProbDgrad2 = ProbDgrad2T<false>;

// dW2_e[d, f] = dy_e^T h_e: A[m=d][k=r] = dy[r][d], B[k=r][n=f] = h[r][f]
struct ProbWgrad2 : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::K;
  static constexpr bool A_KC = false, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  const bf16_t* dY = nullptr; const bf16_t* Hm = nullptr;
  bf16_t* dW2 = nullptr;
  __device__ const bf16_t* a_row(int, int r) const { return dY + (int64_t)r * M; }
  __device__ const bf16_t* b_row(int, int r) const { return Hm + (int64_t)r * N; }
  static constexpr bool STORE16 = true;
  __device__ bf16_t* out_row(int e, int m) const { return dW2 + ((int64_t)e * M + m) * N; }
  __device__ void epilogue4(int e, int m, int n, const float (&v)[4]) const {
    store_bf16x4(dW2 + ((int64_t)e * M + m) * N + n, v);
  }
};

// dx_e = [da | db] [W1_e ; W3_e]: K = 2f, B rows k < f from W1, else W3 (read [k][n=d])
struct ProbDgrad1 : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int f = 0;
  const bf16_t* dab = nullptr; const bf16_t* W1 = nullptr; const bf16_t* W3 = nullptr;
  bf16_t* dX = nullptr;
  __device__ const bf16_t* a_row(int, int m) const { return dab + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int k) const {
    return k < f ? W1 + ((int64_t)e * f + k) * N : W3 + ((int64_t)e * f + (k - f)) * N;
  }
  static constexpr bool K_SPLIT = true;
  __device__ int k_split() const { return f; }
  static constexpr bool STORE16 = true;
  __device__ bf16_t* out_row(int, int m) const { return dX + (int64_t)m * N; }
  __device__ void epilogue4(int, int m, int n, const float (&v)[4]) const { store_bf16x4(dX + (int64_t)m * N + n, v); }
};

// [dW1_e ; dW3_e] [2f, d] = [da | db]_e^T X_e: A[m][k=r] = dab[r][m], B[k=r][n] = x_perm[r][n]
struct ProbWgrad1 : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::K;
  static constexpr bool A_KC = false, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int f = 0;
  const bf16_t* dab = nullptr; const bf16_t* X = nullptr;
  bf16_t* dW1 = nullptr; bf16_t* dW3 = nullptr;
  __device__ const bf16_t* a_row(int, int r) const { return dab + (int64_t)r * M; }
  __device__ const bf16_t* b_row(int, int r) const { return X + (int64_t)r * N; }
  static constexpr bool STORE16 = true;
  __device__ bf16_t* out_row(int e, int m) const {
    return m < f ? dW1 + ((int64_t)e * f + m) * N : dW3 + ((int64_t)e * f + (m - f)) * N;
  }
  __device__ void epilogue4(int e, int m, int n, const float (&v)[4]) const { store_bf16x4(out_row(e, m) + n, v); }
};

// Router scores: logits[t, e] = x[t] . Wr[e] + bias[e]  (single group over T rows)
struct ProbRouterFwd : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = true;
  static constexpr Epi EPI = Epi::Store;
  const bf16_t* X = nullptr; const bf16_t* Wr = nullptr; const float* bias = nullptr;
  float* L = nullptr;
  __device__ const bf16_t* a_row(int, int m) const { return X + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int, int n) const { return Wr + (int64_t)n * K; }
  __device__ void epilogue4(int, int m, int n, const float (&v)[4]) const {
#pragma unroll
    for (int c = 0; c < 4; c++)
      if (n + c < N) L[(int64_t)m * N + n + c] = v[c] + (bias ? bias[n + c] : 0.f);
  }
};

// dx_r = dlogits Wr: A = the bf16 copy of dlogits [T][lda] (experts zero-padded to lda),
// B[k=e][n] = Wr[e][n]
struct ProbRouterDx : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int lda = 0;
  const bf16_t* dL = nullptr; const bf16_t* Wr = nullptr;
  bf16_t* dX = nullptr;
  __device__ const bf16_t* a_row(int, int m) const { return dL + (int64_t)m * lda; }
  __device__ const bf16_t* b_row(int, int k) const { return Wr + (int64_t)k * N; }
  static constexpr bool STORE16 = true;
  __device__ bf16_t* out_row(int, int m) const { return dX + (int64_t)m * N; }
  __device__ void epilogue4(int, int m, int n, const float (&v)[4]) const { store_bf16x4(dX + (int64_t)m * N + n, v); }
};

// Partial router weight gradients: split s of the T rows writes
// part[s][e][i] = sum_{t in split s} dlogits[t, e] x[t, i]; a second kernel sums splits.
struct ProbRouterDwSplit : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::K;
  static constexpr bool A_KC = false, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int lda = 0;
  const bf16_t* dL = nullptr; const bf16_t* X = nullptr;
  float* part = nullptr;
  __device__ const bf16_t* a_row(int, int r) const { return dL + (int64_t)r * lda; }
  __device__ const bf16_t* b_row(int, int r) const { return X + (int64_t)r * N; }
  __device__ void epilogue4(int e, int m, int n, const float (&v)[4]) const {
    *reinterpret_cast<float4*>(part + ((int64_t)e * M + m) * N + n) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Weight gradient of a single group (E == 1) split over the rows: split s writes
// part[s][m][n] = sum_{r in split s} A[r][m] B[r][n] (A [R][M], B [R][N] bf16)
struct ProbWgradSplit : ProbBase {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::K;
  static constexpr bool A_KC = false, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  const bf16_t* A = nullptr; const bf16_t* B = nullptr;
  float* part = nullptr;
  __device__ const bf16_t* a_row(int, int r) const { return A + (int64_t)r * M; }
  __device__ const bf16_t* b_row(int, int r) const { return B + (int64_t)r * N; }
  __device__ void epilogue4(int e, int m, int n, const float (&v)[4]) const {
    *reinterpret_cast<float4*>(part + ((int64_t)e * M + m) * N + n) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

namespace {
// out = sum over splits s (in order) of part[s], rounded to bf16; rows m < split_row go
// to O0 + m * N, the others to O1 + (m - split_row) * N.  Four elements per thread.
__global__ void sum_splits_bf16_kernel(int64_t mn, int N, int nsplit, const float* __restrict__ part, int split_row,
                                       bf16_t* __restrict__ O0, bf16_t* __restrict__ O1) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= mn) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; s++) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)s * mn + i);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  const int64_t m = i / N, n = i % N;
  bf16_t* o = m < split_row ? O0 + m * N + n : O1 + (m - split_row) * N + n;
  const float a[4] = {acc.x, acc.y, acc.z, acc.w};
  store_bf16x4(o, a);
}

// dlogits [T][E] float -> bf16 [T][lda], experts E..lda-1 zero (round to nearest even, as
// the GEMM operand staging always did)
__global__ void dlogits_bf16_kernel(int T, int E, int lda, const float* __restrict__ src, bf16_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * lda) return;
  const int64_t t = i / lda;
  const int e = (int)(i - t * lda);
  dst[i] = e < E ? f2bf(src[t * E + e]) : (bf16_t)0;
}

// dW[i] = sum over splits s (in order) of part[s][i]
__global__ void sum_splits_kernel(int64_t n, int nsplit, const float* __restrict__ part, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int s = 0; s < nsplit; s++) acc += part[(int64_t)s * n + i];
  out[i] = acc;
}
}  // namespace

// ---------------------------------------------------------------------------------------
// Pipelined kernel for bf16 operands.  Each k-step's operand tiles go from global memory
// straight into one of NS (2 to 4) LDS stage buffers, NS - 1 steps ahead of the MFMAs
// (one barrier per k-step).  Loads go through buffer resources that start at a 1 KB
// segment's first row and end at its last valid byte, so rows past a segment end (ragged
// experts, reductions that stop mid-tile) and columns past the matrix edge read as zero
// without any out-of-range access.
//
// LDS tiles are unpadded and XOR-swizzled in 16-byte chunks (see swz): 16 consecutive
// rows read at one logical chunk (K-contiguous tiles, ds_read_b128) or 4 consecutive rows
// read at a pair of chunks (MN-contiguous tiles, ds_read_b64_tr_b16) fall on distinct
// banks of the 64-bank LDS.
// ---------------------------------------------------------------------------------------
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <bool KC, int BMN, int TK, int NW>
struct PipeOperand {
  static constexpr int TILE_BYTES = BMN * TK * 2;    // TK x BMN bf16
  static constexpr int SEGS = TILE_BYTES / 1024;     // one load instruction each
  static constexpr int ROW_BYTES = KC ? TK * 2 : BMN * 2;
  static constexpr int ROWS_PER_SEG = 1024 / ROW_BYTES;
  static constexpr int CPR = ROW_BYTES / 16;         // 16-byte chunks per LDS row
  static_assert(SEGS % NW == 0, "every wave issues the same number of segments");
  static_assert(KC || CPR >= 4, "MN-contiguous tiles need at least 64 columns");
  static constexpr int PER_THREAD = SEGS / NW;       // 1 KB segments per wave

  // physical 16-byte chunk of logical chunk c in tile row r.  16 consecutive rows read
  // at one logical chunk (K-contiguous) or 4 consecutive rows read at a pair of chunks
  // (MN-contiguous, transpose reads) fall on distinct banks of a 64-bank LDS.
  static __device__ __forceinline__ int swz(int r, int c) {
    if constexpr (KC) {
      if constexpr (CPR == 8) return c ^ ((r >> 1) & 7);
      else return c ^ ((r >> 2) & 3);
    } else {
      return c ^ ((4 * (r & 3)) & (CPR - 1));
    }
  }

  // Scalar load state of the operand for the load cursor (kept in scalar registers): per
  // segment of this wave, the address of its first
  // row at the current k-step, the row stride and, for K-contiguous tiles, the bytes it
  // may read.  Rows are mn (K-contiguous tiles) or k (MN-contiguous tiles).  Set up once
  // per tile (begin); each k-step then moves the addresses by one add (next).
  struct Stream {
    const char* ptr[PER_THREAD];
    uint32_t bytes[PER_THREAD];  // K-contiguous: bytes readable from ptr
    uint32_t rb;                 // bytes between consecutive rows
    int k_left;                  // MN-contiguous: rows left from this step to the reduction end
    uint32_t col_bytes;          // MN-contiguous: valid bytes of a row
  };

  // K-contiguous: rows [row0, row_end) valid, k-step starting at column kt
  template <class RowPtr>
  static __device__ __forceinline__ void begin_kc(Stream& st, RowPtr rowptr, int row0, int row_end, int kt, int wave,
                                                  bool live) {
    st.rb = (uint32_t)((rowptr(row0 + 1) - rowptr(row0)) * 2);
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) {
      const int r0 = row0 + (wave + NW * i) * ROWS_PER_SEG;
      st.ptr[i] = reinterpret_cast<const char*>(rowptr(r0) + kt);
      int valid = live ? row_end - r0 : 0;
      valid = valid < 0 ? 0 : (valid > ROWS_PER_SEG ? ROWS_PER_SEG : valid);
      st.bytes[i] = valid > 0 ? (uint32_t)(valid - 1) * st.rb + TK * 2 : 0u;
    }
  }
  // MN-contiguous: k rows [k0, k_end) valid, columns [col0, col_end) valid
  template <class RowPtr>
  static __device__ __forceinline__ void begin_mn(Stream& st, RowPtr rowptr, int k0, int k_end, int col0, int col_end,
                                                  int wave, bool live) {
    st.rb = (uint32_t)((rowptr(k0 + 1) - rowptr(k0)) * 2);
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++)
      st.ptr[i] = reinterpret_cast<const char*>(rowptr(k0 + (wave + NW * i) * ROWS_PER_SEG) + col0);
    st.k_left = live ? k_end - k0 : 0;
    st.col_bytes = (uint32_t)((col_end - col0 < BMN ? col_end - col0 : BMN) * 2);
  }
  // the next k-step of the same rows
  static __device__ __forceinline__ void next(Stream& st) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) st.ptr[i] += KC ? TK * 2 : (int64_t)TK * st.rb;
    if constexpr (!KC) st.k_left -= TK;
  }

  // A tile's loads go straight into LDS (buffer_load ... lds): the 64 16-byte chunks of
  // one wave form one 1 KB segment, lane l landing at segment base + 16 l, and each lane
  // fetches the logical chunk that the swizzle maps there.  The bounds (a buffer resource
  // per segment) are wave-uniform; lanes past the resource's byte count write zeros.
  static __device__ __forceinline__ void dma(const Stream& st, char* lds_tile, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) {
      const int s = wave + NW * i;
      uint32_t bytes;
      if constexpr (KC) {
        bytes = st.bytes[i];
      } else {
        int valid = st.k_left - s * ROWS_PER_SEG;
        valid = valid < 0 ? 0 : (valid > ROWS_PER_SEG ? ROWS_PER_SEG : valid);
        bytes = valid > 0 ? (uint32_t)(valid - 1) * st.rb + st.col_bytes : 0u;
      }
      const int r = lane / CPR, p = lane % CPR;
      const int c = swz(s * ROWS_PER_SEG + r, p);
      const uint32_t voff = (uint32_t)r * st.rb + (uint32_t)(c * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(st.ptr[i], bytes), (lds_void_t*)(lds_tile + s * 1024), 16,
                                               voff, 0, 0, 0);
    }
  }
  // MFMA operand fragment for k-step kk (16 deep): 8 consecutive k of row/column mn0 + lane%32
  static __device__ __forceinline__ bf16x8 frag(const char* lds_tile, int kk, int mn0, int lane) {
    if constexpr (KC) {
      const int r = mn0 + (lane & 31);
      const int c = 2 * kk + (lane >> 5);
      const uint4 q = *reinterpret_cast<const uint4*>(lds_tile + r * ROW_BYTES + (swz(r, c) << 4));
      return __builtin_bit_cast(bf16x8, q);
    } else {
      const int g = lane >> 4, L = lane & 15;
      const int k = 16 * kk + 8 * (g >> 1) + (L >> 2);
      const int b = (mn0 + 16 * (g & 1) + 4 * (L & 3)) * 2;
      const int off = k * ROW_BYTES + (swz(k, b >> 4) << 4) + (b & 15);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_tile + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_tile + off + 4 * ROW_BYTES));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8, v);
    }
  }
};

}  // namespace

// Occupancy target: 8-wave tiles with 2x2 accumulator blocks per wave at a k-depth of 32
// fit 4 waves per SIMD (two workgroups per compute unit) in 128 registers; tiles with
// 4x4 blocks per wave keep their accumulators in AGPRs at one wave per SIMD.  With NL
// loader waves added, the workgroup's waves share the SIMDs at (compute + NL) / 4 each.
template <class Cfg, int TK, int NL>
constexpr int pipe_waves_per_eu() {
  if constexpr (NL > 0) return (Cfg::NT / 64 + NL) / 4;
  return Cfg::WTM * Cfg::WTN >= 16 ? 1 : (TK == 32 && Cfg::WTM * Cfg::WTN <= 4 ? 4 : 2);
}

// Group starts and the tile map live in dynamic LDS sized by the expert count.
static inline size_t pipe_dyn_lds_bytes(int E) { return (size_t)2 * (E + 1) * sizeof(int); }

// NL = 0: every wave loads operands and computes.  NL > 0: the Cfg::NT threads compute
// and NL more waves ("loaders") issue every operand load.  The compute waves then issue no
// load of their own, so nothing makes them wait on the memory counter that their
// epilogue stores also count in: a tile's stores drain while the next tile's MFMAs run.
template <class Cfg, class Prob, int TK, int NS, int NL = 0>
__global__ void __launch_bounds__(Cfg::NT + 64 * NL)
    __attribute__((amdgpu_waves_per_eu(pipe_waves_per_eu<Cfg, TK, NL>()))) grouped_gemm_pipe_kernel(const Prob p) {
  static_assert(NS >= 2 && NS <= 4, "two to four stage buffers");
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT;
  constexpr int WTM = Cfg::WTM, WTN = Cfg::WTN;
  constexpr int NWC = NT / 64;                // waves holding accumulators
  constexpr int NTT = NT + 64 * NL;           // threads of the workgroup
  constexpr int NW = NL > 0 ? NL : NWC;       // waves issuing operand loads
  using OA = PipeOperand<Prob::A_KC, BM, TK, NW>;
  using OB = PipeOperand<Prob::B_KC, BN, TK, NW>;
  constexpr int STAGE_BYTES = OA::TILE_BYTES + OB::TILE_BYTES;
  // NS stage buffers as separate objects: the compiler then tracks the loads into each
  // one separately and waits only for those a read of it depends on
  __shared__ __attribute__((aligned(1024))) char sm0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sm1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sm2[NS >= 3 ? STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char sm3[NS == 4 ? STAGE_BYTES : 16];
  extern __shared__ __attribute__((aligned(16))) int s_dyn[];
  const int E = p.E;
  int* s_map = s_dyn;
  int* s_seg = s_dyn + E + 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / Cfg::WAVES_N, wave_n = wave % Cfg::WAVES_N;
  const int lwave = NL > 0 ? wave - NWC : wave;  // index among the loading waves
  // group starts are read once into LDS: the tile walk then never waits on global loads
  // (a global load there would also drain the operand loads in flight)
  for (int e = tid; e <= E; e += NTT) s_seg[e] = p.seg(e);
  __syncthreads();
  auto seg = [&](int e) { return s_seg[e]; };

  const int total_tiles = build_tile_map<Prob::GROUP, BM, BN, NTT>(s_map, seg, E, p.M, p.N, tid);
  const int G = gridDim.x;
  const int wg = xcd_logical_wg();

  if (wg >= total_tiles) return;  // uniform over the workgroup
  // tile ranges are workgroup-uniform: keep them in scalar registers
  auto tile = [&](int t) {
    TileRange r = tile_at<Prob::GROUP, BM, BN, Prob::N_MAJOR>(t, s_map, seg, E, p.M, p.N, p.K);
    r.e = __builtin_amdgcn_readfirstlane(r.e);
    r.m0 = __builtin_amdgcn_readfirstlane(r.m0);
    r.m_end = __builtin_amdgcn_readfirstlane(r.m_end);
    r.n0 = __builtin_amdgcn_readfirstlane(r.n0);
    r.k_beg = __builtin_amdgcn_readfirstlane(r.k_beg);
    r.k_end = __builtin_amdgcn_readfirstlane(r.k_end);
    return r;
  };

  // The workgroup's tiles form one stream of k-steps: every tile takes
  // max(1, ceil(k range / TK)) steps (a tile with an empty reduction still runs one step
  // on zero operands and stores its zeros).  The load cursor runs NS - 1 steps ahead of
  // the MFMAs across tile boundaries, so the next tile's first stages are in flight while
  // the current tile's epilogue stores.
  struct Cursor {
    int t, k;
    TileRange tr;
  };
  Cursor lc;
  lc.t = wg;
  lc.tr = tile(wg);
  lc.k = lc.tr.k_beg;
  // address streams of the two operands at the load cursor.  The lambdas that set them up
  // and move them are forced inline: a call left out of line keeps the streams in scratch
  // memory (seen with four loader waves, 64-deep steps and a split B operand).
  typename OA::Stream sa;
  typename OB::Stream sb;
  auto begin_streams = [&]() __attribute__((always_inline)) {
    const TileRange& r = lc.tr;
    const bool live = lc.t < total_tiles;
    if constexpr (Prob::A_KC)
      OA::begin_kc(sa, [&](int x) { return p.a_row(r.e, x); }, r.m0, r.m_end, lc.k, lwave, live && lc.k < r.k_end);
    else
      OA::begin_mn(sa, [&](int x) { return p.a_row(r.e, x); }, lc.k, r.k_end, r.m0, r.m_end, lwave, live);
    if constexpr (Prob::B_KC)
      OB::begin_kc(sb, [&](int x) { return p.b_row(r.e, x); }, r.n0, p.N, lc.k, lwave, live && lc.k < r.k_end);
    else
      OB::begin_mn(sb, [&](int x) { return p.b_row(r.e, x); }, lc.k, r.k_end, r.n0, p.N, lwave, live);
  };
  auto advance = [&]() __attribute__((always_inline)) {
    lc.k += TK;
    if (lc.k >= lc.tr.k_end) {
      lc.t += G;
      if (lc.t < total_tiles) lc.tr = tile(lc.t);
      lc.k = lc.tr.k_beg;
      begin_streams();
    } else if (Prob::K_SPLIT && lc.k == p.k_split()) {
      begin_streams();
    } else {
      OA::next(sa);
      OB::next(sb);
    }
  };

  // operands of the load cursor's step go straight into a stage buffer; steps past the
  // reduction or past the last tile read nothing and leave zeros
  auto load_stage = [&](char* base) __attribute__((always_inline)) {
    OA::dma(sa, base, lwave, lane);
    OB::dma(sb, base + OA::TILE_BYTES, lwave, lane);
    advance();
  };
  // this wave's loads into buf have landed (a read of buf makes the compiler wait for
  // exactly those), then every wave meets: buf is complete, and every wave is done with
  // the buffer computed in the previous step
  auto ready = [&](const char* buf) {
    typedef __attribute__((address_space(3))) const volatile int lds_int_t;
    const int v = *(lds_int_t*)(buf + lane * 4);
    asm volatile("s_waitcnt lgkmcnt(0)" ::"v"(v) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // a compute wave beside loader waves only meets them: its reads of the previous buffer
  // were consumed by that step's MFMAs
  auto meet = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 acc[WTM][WTN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < WTM; i++)
#pragma unroll
      for (int j = 0; j < WTN; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
  };
  // MFMAs of one k-step.  Fragments are double-buffered: slice kk+1 is read from LDS
  // before slice kk's MFMAs issue, so its latency runs under them.
  // With loader waves beside 4 x 2 accumulator blocks per wave, the fragments are read one
  // slice at a time (single-buffered) so the workgroup fits three waves per SIMD.
  constexpr bool FRAG1 = NL > 0 && WTM * WTN >= 8;
  auto compute = [&](const char* st) {
    constexpr int KS = TK / 16;
    constexpr int NREAD = (Prob::A_KC ? 1 : 2) * WTM + (Prob::B_KC ? 1 : 2) * WTN;
    if constexpr (FRAG1) {
      bf16x8 af1[WTM], bf1[WTN];
#pragma unroll
      for (int kk = 0; kk < KS; kk++) {
#pragma unroll
        for (int i = 0; i < WTM; i++) af1[i] = OA::frag(st, kk, (wave_m * WTM + i) * 32, lane);
#pragma unroll
        for (int j = 0; j < WTN; j++) bf1[j] = OB::frag(st + OA::TILE_BYTES, kk, (wave_n * WTN + j) * 32, lane);
#pragma unroll
        for (int i = 0; i < WTM; i++)
#pragma unroll
          for (int j = 0; j < WTN; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af1[i], bf1[j], acc[i][j], 0, 0, 0);
      }
#pragma unroll
      for (int kk = 0; kk < KS; kk++) {
        __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, WTM * WTN, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    bf16x8 af[2][WTM], bfr[2][WTN];
    auto read = [&](int kk, int b) {
#pragma unroll
      for (int i = 0; i < WTM; i++) af[b][i] = OA::frag(st, kk, (wave_m * WTM + i) * 32, lane);
#pragma unroll
      for (int j = 0; j < WTN; j++) bfr[b][j] = OB::frag(st + OA::TILE_BYTES, kk, (wave_n * WTN + j) * 32, lane);
    };
    read(0, 0);
#pragma unroll
    for (int kk = 0; kk < KS; kk++) {
      if (kk + 1 < KS) read(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int i = 0; i < WTM; i++)
#pragma unroll
        for (int j = 0; j < WTN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bfr[kk & 1][j], acc[i][j], 0, 0, 0);
    }
    // issue order: slice 0's reads, then per slice the next slice's reads ahead of this
    // slice's MFMAs (LDS reads: mask 0x100, MFMA: mask 0x8)
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
#pragma unroll
    for (int kk = 0; kk < KS; kk++) {
      if (kk + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, WTM * WTN, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto epilogue = [&](const TileRange& tr) { tile_epilogue<Prob, WTM, WTN>(p, acc, tr, wave_m, wave_n, lane); };
  auto steps_of = [&](const TileRange& r) {
    const int n = (r.k_end - r.k_beg + TK - 1) / TK;
    return n < 1 ? 1 : n;
  };

  // compute cursor: tile ct (range ctr), step cs of its ncs steps.  Every wave runs it
  // (loader waves too) so that all of them take the same steps and barriers.
  int ct = wg;
  TileRange ctr = lc.tr;
  int ncs = steps_of(ctr), cs = 0;
  bool done = false;
  // with_acc: the wave holds accumulators, stores the finished tile and clears them
  auto finish_step = [&](bool with_acc) {
    if (++cs == ncs) {
      if (with_acc) epilogue(ctr);
      ct += G;
      if (ct < total_tiles) {
        ctr = tile(ct);
        ncs = steps_of(ctr);
        cs = 0;
        if (with_acc) zero_acc();
      } else {
        done = true;
      }
    }
  };

  // step s is loaded into buffer s % NS, NS - 1 steps ahead; the buffer it overwrites was
  // computed in the step before (every wave is past that step's barrier).  One exit, at
  // the bottom: up to NS - 1 discarded steps run after a workgroup's last tile.
  auto pipeline = [&](auto&& phase) {
    for (;;) {
      if constexpr (NS == 2) {
        phase(sm0, sm1, true);
        phase(sm1, sm0, false);
      } else if constexpr (NS == 3) {
        phase(sm0, sm2, true);
        phase(sm1, sm0, false);
        phase(sm2, sm1, false);
      } else {
        phase(sm0, sm3, true);
        phase(sm1, sm0, false);
        phase(sm2, sm1, false);
        phase(sm3, sm2, false);
      }
      if (done) break;
    }
  };
  auto prologue_loads = [&]() {
    begin_streams();
    load_stage(sm0);  // step 0
    if constexpr (NS >= 3) load_stage(sm1);  // step 1
    if constexpr (NS == 4) load_stage(sm2);
  };
  if constexpr (NL == 0) {
    zero_acc();
    prologue_loads();
    pipeline([&](char* cur, char* next_load, bool first) {
      ready(cur);
      load_stage(next_load);
      compute(cur);
      if (first || !done) finish_step(true);
    });
  } else if (wave >= NWC) {
    // loader: the two roles run separate loops, so no operand load is on a compute
    // wave's path and the compiler puts no memory-counter wait there
    prologue_loads();
    pipeline([&](char* cur, char* next_load, bool first) {
      ready(cur);
      load_stage(next_load);
      if (first || !done) finish_step(false);
    });
  } else {
    zero_acc();
    pipeline([&](char* cur, char*, bool first) {
      meet();
      compute(cur);
      if (first || !done) finish_step(true);
    });
  }
}

// ---------------------------------------------------------------------------------------
// Launchers: tile shape per GEMM (MOE_TILE_<GEMM>=128x256 etc. overrides the default)
// ---------------------------------------------------------------------------------------
enum class Tile { t128x128, t128x256, t256x128, t64x128, t32x128, t256x128w8, t128x256w8, t256x256w8, t256x256w4,
                  t128x256w2, t128x256m1, t192x256w8 };

static bool parse_tile(const char* v, Tile* t) {
  if (!v) return false;
  const struct { const char* s; Tile t; } tab[] = {{"128x128", Tile::t128x128}, {"128x256", Tile::t128x256},
                                                  {"256x128", Tile::t256x128},
                                                  {"64x128", Tile::t64x128},   {"32x128", Tile::t32x128},
                                                  {"256x128w8", Tile::t256x128w8}, {"128x256w8", Tile::t128x256w8},
                                                  {"256x256w8", Tile::t256x256w8}, {"256x256w4", Tile::t256x256w4},
                                                  {"128x256w2", Tile::t128x256w2}, {"128x256m1", Tile::t128x256m1},
                                                  {"192x256w8", Tile::t192x256w8}};
  for (const auto& e : tab)
    if (strcmp(v, e.s) == 0) { *t = e.t; return true; }
  return false;
}

struct TileChoice {
  Tile tile;
  int bk;
  int stages;   // LDS stage buffers: 3, or 4 at a k-depth of 32, or 2 at a k-depth of 64 (where they fit)
  int loaders;  // extra waves that issue every operand load (0, or 4 for 8-wave 128 x 256 and 256 x 256 tiles)
};

// Tile shape, k-depth, stage count and loader waves of one GEMM: MOE_TILE_<NAME> /
// MOE_TILE, MOE_GEMM_BK, MOE_GEMM_STAGES and MOE_GEMM_LOADERS override the defaults chosen
// by measurement on MI355X.
static TileChoice tile_for(const char* name, Tile dflt, int dflt_bk, int dflt_stages = 3, int dflt_loaders = 0) {
  char key[64];
  snprintf(key, sizeof key, "MOE_TILE_%s", name);
  Tile t = dflt;
  if (!parse_tile(tuning_env(key), &t)) parse_tile(tuning_env("MOE_TILE"), &t);
  const char* bk = tuning_env("MOE_GEMM_BK");
  const int b = bk ? atoi(bk) : dflt_bk;
  const char* ns = tuning_env("MOE_GEMM_STAGES");
  const int n = ns ? atoi(ns) : dflt_stages;
  const char* nl = tuning_env("MOE_GEMM_LOADERS");
  const int l = nl ? atoi(nl) : dflt_loaders;
  return TileChoice{t, b == 64 ? 64 : 32, n == 4 ? 4 : (n == 2 ? 2 : 3), l == 4 ? 4 : 0};
}

// Persistent grid: resident workgroups per CU x CUs, capped by the tile bound known on the
// host, rounded to a multiple of the 8 XCDs.
template <class Cfg, class Prob, class Kern>
static hipError_t launch_kernel(Kern kern, const Prob& p, hipStream_t st, size_t dyn_lds, int threads) {
  const int occ = kernel_occupancy(reinterpret_cast<const void*>(kern), threads, dyn_lds);
  int64_t bound;
  const int64_t ntn = (p.N + Cfg::BN - 1) / Cfg::BN;
  if constexpr (Prob::GROUP == Group::M) bound = ((int64_t)p.M / Cfg::BM + p.E) * ntn;
  else bound = (int64_t)p.E * ((p.M + Cfg::BM - 1) / Cfg::BM) * ntn;
  int64_t G = (int64_t)device_cu_count() * occ;
  if (bound < G) G = bound;
  G = ((G + 7) / 8) * 8;
  if (G < 8) G = 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(threads), dyn_lds, st, p);
  return hipGetLastError();
}

template <class Cfg, class Prob, int TK, int NS, int NL = 0>
static hipError_t launch_pipe(const Prob& p, hipStream_t st) {
  // occupancy depends on the dynamic LDS, i.e. on the expert count (cached per size)
  return launch_kernel<Cfg>(grouped_gemm_pipe_kernel<Cfg, Prob, TK, NS, NL>, p, st, pipe_dyn_lds_bytes(p.E),
                            Cfg::NT + 64 * NL);
}

// every problem runs on the pipelined kernel
template <class Cfg, class Prob>
static hipError_t launch_cfg(const Prob& p, hipStream_t st, int bk, int stages, int loaders) {
  static_assert(std::is_same<typename Prob::TA, bf16_t>::value, "bf16 operands");
  // the SwiGLU epilogue pairs each wave's 32-column blocks (a, b): a tile override whose
  // waves hold an odd number of them runs the default tile instead
  if constexpr (Prob::EPI == Epi::SwiGLU && Cfg::WTN % 2 != 0) {
    return launch_cfg<TileCfg<128, 256, 2, 4>>(p, st, bk, stages, loaders);
  } else if constexpr (Cfg::BM == 192) {
    // 192-row tiles (GEMMs grouped along M): 64 deep in two stages, or with loader waves
    // 32 deep in three or four.  The default build compiles them for dgrad1 and dgrad2 (whose
    // defaults use them); another GEMM asking for them runs its default tile.
#ifdef MOE_ALL_TILES
    constexpr bool built = true;
#else
    constexpr bool built = std::is_same<Prob, ProbDgrad1>::value || std::is_same<Prob, ProbDgrad2>::value;
#endif
    if constexpr (!built) {
      return launch_cfg<TileCfg<128, 256, 2, 4>>(p, st, bk, stages, loaders);
    } else if constexpr (Prob::GROUP == Group::M && Cfg::BN == 256 && Cfg::NT == 512) {
      if (loaders == 4) {
        if (bk == 64) return launch_pipe<Cfg, Prob, 64, 2, 4>(p, st);
        if (stages == 3) return launch_pipe<Cfg, Prob, 32, 3, 4>(p, st);
        return launch_pipe<Cfg, Prob, 32, 4, 4>(p, st);
      }
      return launch_pipe<Cfg, Prob, 64, 2>(p, st);
    } else {
      return hipErrorInvalidConfiguration;
    }
  } else {
  // the stage buffers must fit the 160 KB of LDS with room for the tile map
  constexpr bool fits64 = 3 * (Cfg::BM + Cfg::BN) * 64 * 2 <= 152 * 1024;
  constexpr bool fits32x4 = 4 * (Cfg::BM + Cfg::BN) * 32 * 2 <= 152 * 1024;
  constexpr bool fits64x2 = 2 * (Cfg::BM + Cfg::BN) * 64 * 2 <= 152 * 1024;
  // loader waves (GEMMs grouped along M): 8 compute waves with 2 x 2 accumulator blocks
  // each, three stages
  if constexpr (Prob::GROUP == Group::M && Cfg::BM == 128 && Cfg::BN == 256 && Cfg::NT == 512) {
    if (loaders == 4 && stages == 3) {
      if (bk == 64) return launch_pipe<Cfg, Prob, 64, 3, 4>(p, st);
      return launch_pipe<Cfg, Prob, 32, 3, 4>(p, st);
    }
  }
  // loader waves for the 256 x 256 weight-gradient tiles, 32 deep in four stages: the
  // compute waves then issue only their epilogue stores, which no operand load waits behind
  if constexpr (Prob::GROUP == Group::K && Cfg::BM == 256 && Cfg::BN == 256 && Cfg::NT == 512) {
    if (loaders == 4 && bk == 32 && stages == 4) return launch_pipe<Cfg, Prob, 32, 4, 4>(p, st);
  }
  if constexpr (Cfg::BM >= 64 && Cfg::BN >= 64 && fits64x2) {
    if (bk == 64 && stages == 2) return launch_pipe<Cfg, Prob, 64, 2>(p, st);
  }
  if constexpr (Cfg::BM >= 64 && Cfg::BN >= 64) {
    if (bk == 32 || !fits64) {
      if constexpr (fits32x4) {
        if (stages == 4) return launch_pipe<Cfg, Prob, 32, 4>(p, st);
      }
      return launch_pipe<Cfg, Prob, 32, 3>(p, st);
    }
  }
  // the router's scores: one narrow tile per compute unit walks the whole model width, so
  // a fourth stage buffer keeps three 64-deep steps in flight
  constexpr bool fits64x4 = 4 * (Cfg::BM + Cfg::BN) * 64 * 2 <= 152 * 1024;
  if constexpr (std::is_same<Prob, ProbRouterFwd>::value && fits64x4) {
    if (bk == 64 && stages == 4) return launch_pipe<Cfg, Prob, 64, 4>(p, st);
  }
  if constexpr (fits64) return launch_pipe<Cfg, Prob, 64, 3>(p, st);
  return hipErrorInvalidConfiguration;
  }
}

// The default build compiles the tile shapes the defaults use; -DMOE_ALL_TILES adds the
// rest for tuning sweeps (a tile that is not compiled falls back to 128x128).
template <class Prob>
static hipError_t launch(TileChoice c, const Prob& p, hipStream_t st) {
  switch (c.tile) {
    case Tile::t32x128: return launch_cfg<TileCfg<32, 128, 1, 4>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t128x256w8: return launch_cfg<TileCfg<128, 256, 2, 4>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t256x256w8: return launch_cfg<TileCfg<256, 256, 2, 4>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t192x256w8: return launch_cfg<TileCfg<192, 256, 2, 4>>(p, st, c.bk, c.stages, c.loaders);
#ifdef MOE_ALL_TILES
    case Tile::t128x256: return launch_cfg<TileCfg<128, 256, 2, 2>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t256x128: return launch_cfg<TileCfg<256, 128, 2, 2>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t64x128: return launch_cfg<TileCfg<64, 128, 1, 4>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t256x128w8: return launch_cfg<TileCfg<256, 128, 4, 2>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t256x256w4: return launch_cfg<TileCfg<256, 256, 2, 2>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t128x256w2: return launch_cfg<TileCfg<128, 256, 1, 2>>(p, st, c.bk, c.stages, c.loaders);
    case Tile::t128x256m1: return launch_cfg<TileCfg<128, 256, 1, 4>>(p, st, c.bk, c.stages, c.loaders);
#endif
    default: return launch_cfg<TileCfg<128, 128, 2, 2>>(p, st, c.bk, c.stages, c.loaders);
  }
}

// Tiles of the GEMMs grouped along M (forward and data gradients).  Long expert segments
// (1024 rows per expert or more on average) take 256 x 256 tiles, 64 deep, in two stage
// buffers: on MI355X at 2048 rows per expert that is 4-16% faster than 128 x 256 with
// three stages, which stays best for short segments (256 rows per expert).  There, at a
// k-depth of 64, four loader waves beside the eight compute waves take 5-7% off each GEMM
// (the compute waves' epilogue stores no longer wait behind operand loads); at a depth of
// 32 they gained nothing measurable.
static TileChoice m_grouped_tile(const char* name, const GemmShape& s, int short_bk) {
  if ((int64_t)s.R >= (int64_t)1024 * s.E) return tile_for(name, Tile::t256x256w8, 64, 2);
  return tile_for(name, Tile::t128x256w8, short_bk, 3, short_bk == 64 ? 4 : 0);
}

template <bool Q>
static hipError_t gemm1_launch(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* W1,
                               const bf16_t* W3, bf16_t* ab, bf16_t* h, uint8_t* hq, uint8_t* hs, hipStream_t st) {
  ProbGemm1T<Q> p;
  p.M = s.R; p.N = 2 * s.f; p.K = s.d; p.E = s.E; p.offsets = offsets; p.f = s.f;
  p.X = X; p.W1 = W1; p.W3 = W3; p.ab = ab; p.h = h; p.hq = hq; p.hs = hs;
  return launch(m_grouped_tile("GEMM1", s, 64), p, st);
}
hipError_t gemm1_fwd_bf16(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* W1,
                          const bf16_t* W3, bf16_t* ab, bf16_t* h, hipStream_t st, uint8_t* hq, uint8_t* hs) {
  if (hq) return gemm1_launch<true>(s, offsets, X, W1, W3, ab, h, hq, hs, st);
  return gemm1_launch<false>(s, offsets, X, W1, W3, ab, h, nullptr, nullptr, st);
}
hipError_t gemm2_fwd_bf16(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* W2, bf16_t* Y,
                          hipStream_t st) {
  ProbGemm2 p;
  p.M = s.R; p.N = s.d; p.K = s.f; p.E = s.E; p.offsets = offsets;
  p.Hm = H; p.W2 = W2; p.Y = Y;
  return launch(m_grouped_tile("GEMM2", s, 64), p, st);
}
// dgrad2 runs with loader waves at every segment length: its epilogue reads the saved a, b
// of every output, and with the compute waves issuing no operand loads those reads wait
// only on each other (at 4096 and 2048 rows per expert 14% and 9% faster than the 256 x 256
// two-stage tiles without them).  Short segments keep 128 x 256 tiles, 64 deep.  Long ones
// (1024 rows per expert or more on average) take 192 x 256 tiles, 32 deep in three stages,
// so each weight block is read by fewer tiles of an expert: alternating runs on one MI355X,
// 0.215 -> 0.192 ms at E = 8, T = 8192 and 0.934 -> 0.907 ms at E = 32, T = 16384, d = 4096;
// at 512 and 256 rows per expert they measured 3% slower and even.  The variant that also
// writes MXFP8 rows of [da | db] keeps the 128 x 256 tiles (on 192 x 256 its epilogue took
// 1.74 ms against 1.02 at E = 32, T = 16384, d = 4096).
template <bool Q>
static hipError_t dgrad2_launch(const GemmShape& s, const int* offsets, const bf16_t* dY, const bf16_t* W2,
                                const bf16_t* ab, bf16_t* dab, uint8_t* dq, uint8_t* ds, hipStream_t st) {
  ProbDgrad2T<Q> p;
  p.M = s.R; p.N = s.f; p.K = s.d; p.E = s.E; p.offsets = offsets;
  p.dY = dY; p.W2 = W2; p.ab = ab; p.dab = dab; p.dq = dq; p.ds = ds;
  if (!Q && (int64_t)s.R >= (int64_t)1024 * s.E)
    return launch(tile_for("DGRAD2", Tile::t192x256w8, 32, 3, 4), p, st);
  return launch(tile_for("DGRAD2", Tile::t128x256w8, 64, 3, 4), p, st);
}
hipError_t dgrad2_bf16(const GemmShape& s, const int* offsets, const bf16_t* dY, const bf16_t* W2,
                       const bf16_t* ab, bf16_t* dab, hipStream_t st, uint8_t* dq, uint8_t* ds) {
  if (dq) return dgrad2_launch<true>(s, offsets, dY, W2, ab, dab, dq, ds, st);
  return dgrad2_launch<false>(s, offsets, dY, W2, ab, dab, nullptr, nullptr, st);
}
// Single-group weight gradients: with one expert the output has few tiles (64 for
// 2048 x 2048 at 256 x 256), so the reduction over the R rows is split to give about two
// tiles per CU of a 256-CU device (splits of at least 512 rows); partial sums go to ws and
// are added in split order.  Host-only arithmetic.
static int wgrad_single_splits(int R, int M, int N) {
  const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int s = (512 + tiles - 1) / tiles;
  const int max_s = R / 512;
  if (s > max_s) s = max_s;
  return s < 1 ? 1 : s;
}
size_t wgrad_split_workspace_bytes(const GemmShape& s) {
  if (s.E != 1) return 0;
  const int s1 = wgrad_single_splits(s.R, 2 * s.f, s.d), s2 = wgrad_single_splits(s.R, s.d, s.f);
  const size_t a = s1 > 1 ? (size_t)s1 * 2 * s.f * s.d * sizeof(float) : 0;
  const size_t b = s2 > 1 ? (size_t)s2 * s.d * s.f * sizeof(float) : 0;
  return a > b ? a : b;
}
static hipError_t wgrad_split(int R, int M, int N, int nsplit, const bf16_t* A, const bf16_t* B, float* part,
                              int split_row, bf16_t* O0, bf16_t* O1, hipStream_t st) {
  const int seg_len = (R + nsplit - 1) / nsplit;
  ProbWgradSplit p;
  p.M = M; p.N = N; p.K = R; p.E = (R + seg_len - 1) / seg_len; p.seg_len = seg_len; p.seg_total = R;
  p.A = A; p.B = B; p.part = part;
  hipError_t err = launch(tile_for("WGRAD_SPLIT", Tile::t256x256w8, 32, 4), p, st);
  if (err != hipSuccess) return err;
  const int64_t mn = (int64_t)M * N;
  hipLaunchKernelGGL(sum_splits_bf16_kernel, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, st, mn, N, p.E,
                     part, split_row, O0, O1);
  return hipGetLastError();
}

// Weight-gradient tiles: 256 x 256, 32 deep, four stage buffers.  With 512 or more rows per
// expert on average, four loader waves issue every operand load, so the compute waves' gradient
// stores hold back no load wait: 8-10% faster on both weight gradients at 512, 2048 and 4096
// rows per expert (E = 128, T = 16384; E = 32, d = 4096; E = 8); at 256 rows they gain nothing.
static TileChoice wgrad_tile(const char* name, const GemmShape& s) {
  return tile_for(name, Tile::t256x256w8, 32, 4, (int64_t)s.R >= (int64_t)512 * s.E ? 4 : 0);
}

hipError_t wgrad2_bf16(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* dY, bf16_t* dW2,
                       void* ws, hipStream_t st) {
  if (s.E == 1 && ws) {
    const int ns = wgrad_single_splits(s.R, s.d, s.f);
    if (ns > 1) return wgrad_split(s.R, s.d, s.f, ns, dY, H, static_cast<float*>(ws), s.d, dW2, dW2, st);
  }
  ProbWgrad2 p;
  p.M = s.d; p.N = s.f; p.K = s.R; p.E = s.E; p.offsets = offsets;
  p.dY = dY; p.Hm = H; p.dW2 = dW2;
  return launch(wgrad_tile("WGRAD2", s), p, st);
}
// dgrad1 takes 192 x 256 tiles, 32 deep in three stages, with four loader waves, at every
// segment length: each weight block is then read by ceil(rows / 192) tiles of an expert
// instead of ceil(rows / 128), and the compute waves' stores wait on no operand load.
// Against its former tiles (128 x 256 without loaders for short segments, 256 x 256 64 deep
// in two stages for long ones), alternating runs on one MI355X: 0.399 -> 0.393 ms at E = 128,
// T = 8192; 0.669 -> 0.620 at E = 128, T = 16384 (uniform routing); 0.329 -> 0.289 at E = 8;
// 1.626 -> 1.538 at E = 32, T = 16384, d = 4096.
hipError_t dgrad1_bf16(const GemmShape& s, const int* offsets, const bf16_t* dab, const bf16_t* W1,
                       const bf16_t* W3, bf16_t* dX, hipStream_t st) {
  ProbDgrad1 p;
  p.M = s.R; p.N = s.d; p.K = 2 * s.f; p.E = s.E; p.offsets = offsets; p.f = s.f;
  p.dab = dab; p.W1 = W1; p.W3 = W3; p.dX = dX;
  return launch(tile_for("DGRAD1", Tile::t192x256w8, 32, 3, 4), p, st);
}
hipError_t wgrad1_bf16(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* dab, bf16_t* dW1,
                       bf16_t* dW3, void* ws, hipStream_t st) {
  if (s.E == 1 && ws) {
    const int ns = wgrad_single_splits(s.R, 2 * s.f, s.d);
    if (ns > 1) return wgrad_split(s.R, 2 * s.f, s.d, ns, dab, X, static_cast<float*>(ws), s.f, dW1, dW3, st);
  }
  ProbWgrad1 p;
  p.M = 2 * s.f; p.N = s.d; p.K = s.R; p.E = s.E; p.offsets = offsets; p.f = s.f;
  p.dab = dab; p.X = X; p.dW1 = dW1; p.dW3 = dW3;
  return launch(wgrad_tile("WGRAD1", s), p, st);
}
hipError_t router_fwd_bf16(int T, int d, int E, const bf16_t* X, const bf16_t* Wr, const float* bias, float* L,
                           hipStream_t st) {
  ProbRouterFwd p;
  p.M = T; p.N = E; p.K = d; p.E = 1; p.seg_len = T; p.seg_total = T;
  p.X = X; p.Wr = Wr; p.bias = bias; p.L = L;
  return launch(tile_for("ROUTER_FWD", Tile::t32x128, 64, 4), p, st);
}
// Split count of the router weight gradient: about 256 output tiles in flight (one per
// compute unit of a 256-CU device), splits of at least 64 rows.  At T = 8192, d = 2048,
// E = 128 that is 16 splits of 512 rows: the backward took 54.6 us against 61.6 us with
// 32 splits (half the partial sums to write and add).  Host-only arithmetic.
int router_dw_splits(int T, int d, int E) {
  const int tiles = ((E + 127) / 128) * ((d + 127) / 128);
  int s = (256 + tiles - 1) / tiles;
  const int max_s = (T + 63) / 64;
  if (s > max_s) s = max_s;
  return s < 1 ? 1 : s;
}
int router_lda(int E) { return (E + 63) / 64 * 64; }
static size_t al256(size_t b) { return (b + 255) / 256 * 256; }
size_t router_dw_workspace_bytes(int T, int d, int E) {
  return al256((size_t)T * router_lda(E) * sizeof(bf16_t)) + (size_t)router_dw_splits(T, d, E) * E * d * sizeof(float);
}
// dx_r = dlogits Wr (skipped when dX is null) and dWr = dlogits^T x through the bf16 copy of
// dlogits at the start of ws (split partials of dWr after it)
hipError_t router_bwd_bf16(int T, int d, int E, const float* dL, const bf16_t* Wr, const bf16_t* X, bf16_t* dX,
                           float* dW, void* ws, hipStream_t st) {
  const int lda = router_lda(E);
  bf16_t* dLb = static_cast<bf16_t*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + al256((size_t)T * lda * sizeof(bf16_t)));
  hipError_t err;
  if (T > 0) {
    const int64_t n = (int64_t)T * lda;
    hipLaunchKernelGGL(dlogits_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, T, E, lda, dL, dLb);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (dX) {  // null: the caller folds dx_r into the un-permute (unpermute_router_rows)
      ProbRouterDx p;
      p.M = T; p.N = d; p.K = E; p.E = 1; p.seg_len = T; p.seg_total = T;
      p.lda = lda; p.dL = dLb; p.Wr = Wr; p.dX = dX;
      if ((err = launch(tile_for("ROUTER_DX", Tile::t128x256w8, 64), p, st)) != hipSuccess) return err;
    }
  }
  int ns = router_dw_splits(T, d, E);
  const int seg_len = ((T + ns - 1) / ns + 63) / 64 * 64;
  ns = T == 0 ? 1 : (T + seg_len - 1) / seg_len;
  ProbRouterDwSplit q;
  q.M = E; q.N = d; q.K = T; q.E = ns; q.seg_len = seg_len; q.seg_total = T;
  q.lda = lda; q.dL = dLb; q.X = X; q.part = ns == 1 ? dW : part;
  if ((err = launch(tile_for("ROUTER_DW", Tile::t128x128, 64), q, st)) != hipSuccess || ns == 1) return err;
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, ns, part, dW);
  return hipGetLastError();
}

}  // namespace moe
