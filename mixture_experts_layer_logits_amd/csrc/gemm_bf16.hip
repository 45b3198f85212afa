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
// Tiles are BM x BN with BK = 64, staged through LDS in two buffers.  An operand whose
// reduction axis is contiguous in memory ("K-contiguous") is kept [mn][k] in LDS and
// read with 16-byte ds_read_b128; an operand contiguous along M or N is kept [k][mn]
// as loaded and read with the gfx950 transpose read ds_read_b64_tr_b16, so no operand
// is ever transposed in HBM.  MFMA: v_mfma_f32_32x32x16_bf16 (lane l holds row l%32,
// k = 8*(l/32)..+7 of A; column l%32 of B; accumulator row 8*(i/4)+4*(l/32)+i%4).
#include "common.h"
#include "gemm.h"

namespace moe {

namespace {

constexpr int BK = 64;
constexpr int KC_STRIDE = BK + 8;  // LDS row stride (elements) of a K-contiguous tile

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

__device__ __forceinline__ uint4 pack8(const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; i++) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Two transpose reads give one lane 8 consecutive k of one m/n column of a [k][mn] tile.
__device__ __forceinline__ bf16x8 read_mn_frag(const bf16_t* tile, int stride, int k0, int mn0, int lane) {
  const int g = lane >> 4, L = lane & 15;
  const int k = k0 + 8 * (g >> 1) + (L >> 2);
  const int mn = mn0 + 16 * (g & 1) + 4 * (L & 3);
  const bf16_t* p0 = tile + k * stride + mn;
  const bf16_t* p1 = p0 + 4 * stride;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 read_k_frag(const bf16_t* tile, int k0, int mn0, int lane) {
  const bf16_t* p = tile + (mn0 + (lane & 31)) * KC_STRIDE + k0 + 8 * (lane >> 5);
  uint4 q = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, q);
}

// ---------------------------------------------------------------------------------------
// Operand staging.  A "chunk" is 8 consecutive elements along the contiguous axis.
// ---------------------------------------------------------------------------------------
template <typename T, bool KC, int BMN, int NT>
struct Stager {
  // K-contiguous: tile rows = mn (BMN), 8 chunks per row.  MN-contiguous: tile rows = k
  // (BK), BMN/8 chunks per row.
  static constexpr int CHUNKS = BMN * BK / 8;
  static constexpr int PER_THREAD = CHUNKS / NT;
  static constexpr int LDS_ELEMS = KC ? BMN * KC_STRIDE : BK * (BMN + 16);
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly over the workgroup");
  uint4 reg[PER_THREAD];

  // rowptr(mn) returns the address of element (mn, k=0) for K-contiguous operands, or
  // (k, mn=0) for MN-contiguous ones; validity is checked by the caller-provided bounds.
  template <class RowPtr>
  __device__ __forceinline__ void load(RowPtr rowptr, int mn0, int mn_end, int k0, int k_end, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) {
      const int c = tid + i * NT;
      if constexpr (KC) {
        const int r = c >> 3, kc = (c & 7) * 8;
        const int mn = mn0 + r, k = k0 + kc;
        if constexpr (sizeof(T) == 2) {
          reg[i] = (mn < mn_end && k + 8 <= k_end) ? *reinterpret_cast<const uint4*>(rowptr(mn) + k) : zero4();
        } else {
          float v[8];
          const T* p = rowptr(mn < mn_end ? mn : mn0);
#pragma unroll
          for (int j = 0; j < 8; j++) v[j] = (mn < mn_end && k + j < k_end) ? (float)p[k + j] : 0.f;
          reg[i] = pack8(v);
        }
      } else {
        constexpr int CPR = BMN / 8;
        const int r = c / CPR, mc = (c % CPR) * 8;
        const int k = k0 + r, mn = mn0 + mc;
        if constexpr (sizeof(T) == 2) {
          reg[i] = (k < k_end && mn + 8 <= mn_end) ? *reinterpret_cast<const uint4*>(rowptr(k) + mn) : zero4();
        } else {
          float v[8];
          const T* p = rowptr(k < k_end ? k : k0);
#pragma unroll
          for (int j = 0; j < 8; j++) v[j] = (k < k_end && mn + j < mn_end) ? (float)p[mn + j] : 0.f;
          reg[i] = pack8(v);
        }
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) {
      const int c = tid + i * NT;
      int off;
      if constexpr (KC) {
        off = (c >> 3) * KC_STRIDE + (c & 7) * 8;
      } else {
        constexpr int CPR = BMN / 8;
        off = (c / CPR) * (BMN + 16) + (c % CPR) * 8;
      }
      *reinterpret_cast<uint4*>(lds + off) = reg[i];
    }
  }
  static __device__ __forceinline__ bf16x8 frag(const bf16_t* lds, int kk, int mn0, int lane) {
    if constexpr (KC) return read_k_frag(lds, kk, mn0, lane);
    else return read_mn_frag(lds, BMN + 16, kk, mn0, lane);
  }
};

}  // namespace

// ---------------------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------------------
template <class Cfg, class Prob>
__global__ void __launch_bounds__(Cfg::NT) grouped_gemm_kernel(const Prob p) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT;
  constexpr int WTM = Cfg::WTM, WTN = Cfg::WTN;
  using SA = Stager<typename Prob::TA, Prob::A_KC, BM, NT>;
  using SB = Stager<bf16_t, Prob::B_KC, BN, NT>;
  __shared__ __attribute__((aligned(16))) bf16_t lds_a[2][SA::LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t lds_b[2][SB::LDS_ELEMS];
  // GROUP_M: first m-tile of each expert; GROUP_K: experts by descending row count
  __shared__ int s_map[kMaxExperts + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_m = wave / Cfg::WAVES_N, wave_n = wave % Cfg::WAVES_N;
  const int E = p.E;
  // segment e spans [seg(e), seg(e+1)); without offsets there is one segment over all rows
  const int total_rows = Prob::GROUP == Group::M ? p.M : p.K;
  auto seg = [&](int e) { return p.offsets ? p.offsets[e] : (e == 0 ? 0 : total_rows); };

  // ---- tile map
  int total_tiles;
  const int ntn = (p.N + BN - 1) / BN;
  if constexpr (Prob::GROUP == Group::M) {
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < E; base += kWave) {
        const int e = base + lane;
        const int x = e < E ? (seg(e + 1) - seg(e) + BM - 1) / BM : 0;
        int incl = x;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += y;
        }
        if (e < E) s_map[e] = carry + incl - x;
        carry += __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) s_map[E] = carry;
    }
    __syncthreads();
    total_tiles = s_map[E] * ntn;
  } else {
    // order experts by descending row count (ties: lower id first) so the longest
    // reductions start first; rank by counting
    for (int e = tid; e < E; e += NT) {
      const int ce = seg(e + 1) - seg(e);
      int rank = 0;
      for (int o = 0; o < E; o++) {
        const int co = seg(o + 1) - seg(o);
        rank += (co > ce) || (co == ce && o < e);
      }
      s_map[rank] = e;
    }
    __syncthreads();
    total_tiles = E * ((p.M + BM - 1) / BM) * ntn;
  }

  // ---- XCD-aware persistent schedule: consecutive logical workgroups share an XCD
  // (hardware dispatches workgroup b to XCD b % 8), and consecutive tiles share operands.
  const int G = gridDim.x;
  const int wg = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;

  SA sa;
  SB sb;
  for (int t = wg; t < total_tiles; t += G) {
    int e, m0, m_end, n0, k_beg, k_end;
    if constexpr (Prob::GROUP == Group::M) {
      const int mt = t / ntn;
      n0 = (t % ntn) * BN;
      int lo = 0, hi = E;  // largest e with s_map[e] <= mt
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_map[mid] <= mt) lo = mid; else hi = mid;
      }
      e = lo;
      m0 = seg(e) + (mt - s_map[e]) * BM;
      m_end = seg(e + 1);
      k_beg = 0;
      k_end = p.K;
    } else {
      const int mtn = (p.M + BM - 1) / BM;
      const int per_e = mtn * ntn;
      e = s_map[t / per_e];
      const int rem = t % per_e;
      m0 = (rem / ntn) * BM;
      n0 = (rem % ntn) * BN;
      m_end = p.M;
      k_beg = seg(e);
      k_end = seg(e + 1);
    }

    f32x16 acc[WTM][WTN];
#pragma unroll
    for (int i = 0; i < WTM; i++)
#pragma unroll
      for (int j = 0; j < WTN; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    auto load_stage = [&](int kt) {
      if constexpr (Prob::A_KC) sa.load([&](int m) { return p.a_row(e, m); }, m0, m_end, kt, k_end, tid);
      else sa.load([&](int k) { return p.a_row(e, k); }, m0, m_end, kt, k_end, tid);
      if constexpr (Prob::B_KC) sb.load([&](int n) { return p.b_row(e, n); }, n0, p.N, kt, k_end, tid);
      else sb.load([&](int k) { return p.b_row(e, k); }, n0, p.N, kt, k_end, tid);
    };

    if (k_beg < k_end) {
      load_stage(k_beg);
      sa.store(lds_a[0], tid);
      sb.store(lds_b[0], tid);
      __syncthreads();
      int cur = 0;
      for (int kt = k_beg; kt < k_end; kt += BK) {
        const bool more = kt + BK < k_end;
        if (more) load_stage(kt + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
          bf16x8 af[WTM], bfr[WTN];
#pragma unroll
          for (int i = 0; i < WTM; i++) af[i] = SA::frag(lds_a[cur], kk, (wave_m * WTM + i) * 32, lane);
#pragma unroll
          for (int j = 0; j < WTN; j++) bfr[j] = SB::frag(lds_b[cur], kk, (wave_n * WTN + j) * 32, lane);
#pragma unroll
          for (int i = 0; i < WTM; i++)
#pragma unroll
            for (int j = 0; j < WTN; j++)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
          sa.store(lds_a[cur ^ 1], tid);
          sb.store(lds_b[cur ^ 1], tid);
        }
        __syncthreads();
        cur ^= 1;
      }
    }

    // ---- epilogue straight from the accumulators
#pragma unroll
    for (int i = 0; i < WTM; i++) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = m0 + (wave_m * WTM + i) * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m >= m_end) continue;
        if constexpr (Prob::EPI == Epi::SwiGLU) {
#pragma unroll
          for (int j = 0; j < WTN; j += 2) {
            const int hcol = n0 / 2 + ((wave_n * WTN + j) >> 1) * 32 + (lane & 31);
            p.epilogue_swiglu(m, hcol, acc[i][j][r], acc[i][j + 1][r]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < WTN; j++) {
            const int n = n0 + (wave_n * WTN + j) * 32 + (lane & 31);
            if (n < p.N) p.epilogue(e, m, n, acc[i][j][r]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Problem descriptions (operand addressing + epilogue) for each GEMM of the layer
// ---------------------------------------------------------------------------------------
// Forward GEMM1 with the SwiGLU epilogue: [a | b] = X_e [W1_e | W3_e]^T, the B tile's
// 32-column blocks alternate W1 / W3 rows so each wave holds a and b of the same column.
struct ProbGemm1 {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = true;
  static constexpr Epi EPI = Epi::SwiGLU;
  int M, N, K, E, f;
  const int* offsets;
  const bf16_t* X; const bf16_t* W1; const bf16_t* W3;
  bf16_t* ab; bf16_t* h;
  __device__ const bf16_t* a_row(int, int m) const { return X + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int n) const {
    const int blk = n >> 5, col = (blk >> 1) * 32 + (n & 31);
    const bf16_t* W = (blk & 1) ? W3 : W1;
    return W + ((int64_t)e * f + col) * K;
  }
  __device__ void epilogue_swiglu(int m, int hcol, float a, float b) const {
    bf16_t* abr = ab + (int64_t)m * 2 * f;
    abr[hcol] = f2bf(a);
    abr[f + hcol] = f2bf(b);
    h[(int64_t)m * f + hcol] = f2bf(a * sigmoidf_(a) * b);
  }
  __device__ void epilogue(int, int, int, float) const {}
};

// y_perm = h W2_e^T
struct ProbGemm2 {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = true;
  static constexpr Epi EPI = Epi::Store;
  int M, N, K, E;
  const int* offsets;
  const bf16_t* Hm; const bf16_t* W2;
  bf16_t* Y;
  __device__ const bf16_t* a_row(int, int m) const { return Hm + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int n) const { return W2 + ((int64_t)e * N + n) * K; }
  __device__ void epilogue(int, int m, int n, float v) const { Y[(int64_t)m * N + n] = f2bf(v); }
};

// dh = dy_e W2_e (B = W2_e read [k=d][n=f]) with the SwiGLU-gradient epilogue
struct ProbDgrad2 {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = false;
  static constexpr Epi EPI = Epi::DSwiGLU;
  int M, N, K, E;  // N = f, K = d
  const int* offsets;
  const bf16_t* dY; const bf16_t* W2; const bf16_t* ab;
  bf16_t* dab;
  __device__ const bf16_t* a_row(int, int m) const { return dY + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int k) const { return W2 + ((int64_t)e * K + k) * N; }
  __device__ void epilogue(int, int m, int n, float dh) const {
    const bf16_t* abr = ab + (int64_t)m * 2 * N;
    const float a = bf2f(abr[n]), b = bf2f(abr[N + n]);
    const float s = sigmoidf_(a);
    bf16_t* o = dab + (int64_t)m * 2 * N;
    o[n] = f2bf(dh * b * s * (1.f + a * (1.f - s)));
    o[N + n] = f2bf(dh * a * s);
  }
};

// dW2_e[d, f] = dy_e^T h_e: A[m=d][k=r] = dy[r][d], B[k=r][n=f] = h[r][f]
struct ProbWgrad2 {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::K;
  static constexpr bool A_KC = false, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int M, N, K, E;  // M = d, N = f
  const int* offsets;
  const bf16_t* dY; const bf16_t* Hm;
  bf16_t* dW2;
  __device__ const bf16_t* a_row(int, int r) const { return dY + (int64_t)r * M; }
  __device__ const bf16_t* b_row(int, int r) const { return Hm + (int64_t)r * N; }
  __device__ void epilogue(int e, int m, int n, float v) const { dW2[((int64_t)e * M + m) * N + n] = f2bf(v); }
};

// dx_e = [da | db] [W1_e ; W3_e]: K = 2f, B rows k < f from W1, else W3 (read [k][n=d])
struct ProbDgrad1 {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int M, N, K, E, f;  // N = d, K = 2f
  const int* offsets;
  const bf16_t* dab; const bf16_t* W1; const bf16_t* W3;
  bf16_t* dX;
  __device__ const bf16_t* a_row(int, int m) const { return dab + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int e, int k) const {
    return k < f ? W1 + ((int64_t)e * f + k) * N : W3 + ((int64_t)e * f + (k - f)) * N;
  }
  __device__ void epilogue(int, int m, int n, float v) const { dX[(int64_t)m * N + n] = f2bf(v); }
};

// [dW1_e ; dW3_e] [2f, d] = [da | db]_e^T X_e: A[m][k=r] = dab[r][m], B[k=r][n] = x_perm[r][n]
struct ProbWgrad1 {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::K;
  static constexpr bool A_KC = false, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int M, N, K, E, f;  // M = 2f, N = d
  const int* offsets;
  const bf16_t* dab; const bf16_t* X;
  bf16_t* dW1; bf16_t* dW3;
  __device__ const bf16_t* a_row(int, int r) const { return dab + (int64_t)r * M; }
  __device__ const bf16_t* b_row(int, int r) const { return X + (int64_t)r * N; }
  __device__ void epilogue(int e, int m, int n, float v) const {
    bf16_t* W = m < f ? dW1 + ((int64_t)e * f + m) * N : dW3 + ((int64_t)e * f + (m - f)) * N;
    W[n] = f2bf(v);
  }
};

// Router scores: logits[t, e] = x[t] . Wr[e] + bias[e]  (single group over T rows)
struct ProbRouterFwd {
  using TA = bf16_t;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = true;
  static constexpr Epi EPI = Epi::Store;
  int M, N, K, E;  // M = T, N = experts, K = d; E = 1 group
  const int* offsets;
  const bf16_t* X; const bf16_t* Wr; const float* bias;
  float* L;
  __device__ const bf16_t* a_row(int, int m) const { return X + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int, int n) const { return Wr + (int64_t)n * K; }
  __device__ void epilogue(int, int m, int n, float v) const { L[(int64_t)m * N + n] = v + (bias ? bias[n] : 0.f); }
};

// dx_r = dlogits Wr: A = dlogits [T][E] float (rounded to bf16 on staging), B[k=e][n] = Wr[e][n]
struct ProbRouterDx {
  using TA = float;
  static constexpr Group GROUP = Group::M;
  static constexpr bool A_KC = true, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int M, N, K, E;  // M = T, N = d, K = experts
  const int* offsets;
  const float* dL; const bf16_t* Wr;
  bf16_t* dX;
  __device__ const float* a_row(int, int m) const { return dL + (int64_t)m * K; }
  __device__ const bf16_t* b_row(int, int k) const { return Wr + (int64_t)k * N; }
  __device__ void epilogue(int, int m, int n, float v) const { dX[(int64_t)m * N + n] = f2bf(v); }
};

// dWr[e, i] = sum_t dlogits[t, e] x[t, i]: one group spanning all T rows
struct ProbRouterDw {
  using TA = float;
  static constexpr Group GROUP = Group::K;
  static constexpr bool A_KC = false, B_KC = false;
  static constexpr Epi EPI = Epi::Store;
  int M, N, K, E;  // M = experts, N = d
  const int* offsets;
  const float* dL; const bf16_t* X;
  float* dW;
  __device__ const float* a_row(int, int r) const { return dL + (int64_t)r * M; }
  __device__ const bf16_t* b_row(int, int r) const { return X + (int64_t)r * N; }
  __device__ void epilogue(int, int m, int n, float v) const { dW[(int64_t)m * N + n] = v; }
};

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
using Cfg128 = TileCfg<128, 128, 2, 2>;

template <class Cfg, class Prob>
static hipError_t launch(const Prob& p, int tile_bound, hipStream_t st) {
  int G = device_cu_count() * 2;
  if (tile_bound < G) G = tile_bound;
  G = ((G + 7) / 8) * 8;
  if (G < 8) G = 8;
  hipLaunchKernelGGL((grouped_gemm_kernel<Cfg, Prob>), dim3(G), dim3(Cfg::NT), 0, st, p);
  return hipGetLastError();
}

static int tiles_m_bound(int R, int E, int BM, int N, int BN) {
  int64_t b = ((int64_t)R / BM + E) * ((N + BN - 1) / BN);
  return b > (1 << 30) ? (1 << 30) : (int)b;
}

hipError_t gemm1_fwd_bf16(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* W1,
                          const bf16_t* W3, bf16_t* ab, bf16_t* h, hipStream_t st) {
  ProbGemm1 p{s.R, 2 * s.f, s.d, s.E, s.f, offsets, X, W1, W3, ab, h};
  return launch<Cfg128>(p, tiles_m_bound(s.R, s.E, Cfg128::BM, p.N, Cfg128::BN), st);
}
hipError_t gemm2_fwd_bf16(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* W2, bf16_t* Y,
                          hipStream_t st) {
  ProbGemm2 p{s.R, s.d, s.f, s.E, offsets, H, W2, Y};
  return launch<Cfg128>(p, tiles_m_bound(s.R, s.E, Cfg128::BM, p.N, Cfg128::BN), st);
}
hipError_t dgrad2_bf16(const GemmShape& s, const int* offsets, const bf16_t* dY, const bf16_t* W2,
                       const bf16_t* ab, bf16_t* dab, hipStream_t st) {
  ProbDgrad2 p{s.R, s.f, s.d, s.E, offsets, dY, W2, ab, dab};
  return launch<Cfg128>(p, tiles_m_bound(s.R, s.E, Cfg128::BM, p.N, Cfg128::BN), st);
}
hipError_t wgrad2_bf16(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* dY, bf16_t* dW2,
                       hipStream_t st) {
  ProbWgrad2 p{s.d, s.f, s.R, s.E, offsets, dY, H, dW2};
  int bound = s.E * ((s.d + 127) / 128) * ((s.f + 127) / 128);
  return launch<Cfg128>(p, bound, st);
}
hipError_t dgrad1_bf16(const GemmShape& s, const int* offsets, const bf16_t* dab, const bf16_t* W1,
                       const bf16_t* W3, bf16_t* dX, hipStream_t st) {
  ProbDgrad1 p{s.R, s.d, 2 * s.f, s.E, s.f, offsets, dab, W1, W3, dX};
  return launch<Cfg128>(p, tiles_m_bound(s.R, s.E, Cfg128::BM, p.N, Cfg128::BN), st);
}
hipError_t wgrad1_bf16(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* dab, bf16_t* dW1,
                       bf16_t* dW3, hipStream_t st) {
  ProbWgrad1 p{2 * s.f, s.d, s.R, s.E, s.f, offsets, dab, X, dW1, dW3};
  int bound = s.E * ((2 * s.f + 127) / 128) * ((s.d + 127) / 128);
  return launch<Cfg128>(p, bound, st);
}
hipError_t router_fwd_bf16(int T, int d, int E, const bf16_t* X, const bf16_t* Wr, const float* bias, float* L,
                           hipStream_t st) {
  ProbRouterFwd p{T, E, d, 1, nullptr, X, Wr, bias, L};
  return launch<Cfg128>(p, tiles_m_bound(T, 1, 128, E, 128), st);
}
hipError_t router_dx_bf16(int T, int d, int E, const float* dL, const bf16_t* Wr, bf16_t* dX, hipStream_t st) {
  ProbRouterDx p{T, d, E, 1, nullptr, dL, Wr, dX};
  return launch<Cfg128>(p, tiles_m_bound(T, 1, 128, d, 128), st);
}
hipError_t router_dw_bf16(int T, int d, int E, const float* dL, const bf16_t* X, float* dW, hipStream_t st) {
  ProbRouterDw p{E, d, T, 1, nullptr, dL, X, dW};
  int bound = ((E + 127) / 128) * ((d + 127) / 128);
  return launch<Cfg128>(p, bound, st);
}

}  // namespace moe
