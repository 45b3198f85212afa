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
#include "tilemap.h"

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

// Transposing quantiser: column c of the rows of segment e (blocks of 32 rows, restarting
// at every segment start, a segment's last block zero-padded) goes to output row c:
//   codes  q[qbase(e) + c * ldq + (r - start_e)],   scales s[sbase(e) + c * lds + (r - start_e) / 32]
// Padded mode (routed activations): segments are the expert row ranges seg[e]..seg[e+1];
//   output segment e starts at P_e = sum_{e'<e} roundup(n_e', 128), rows of the padding get
//   zero codes and zero-block scales.  Uniform mode (weights): segment e is rows
//   [e * len, (e + 1) * len) and starts at e * q_seg + col_off (scales e * s_seg + col_off / 32).
struct TransQ {
  const bf16_t* src;
  int64_t ld_src;
  int cols;
  const int32_t* seg;  // padded mode; nullptr for uniform mode
  int nseg;
  int len;             // uniform mode segment length (a multiple of 32)
  uint8_t* q;
  int64_t ldq, q_seg;
  uint8_t* s;
  int64_t lds, s_seg;
  int col_off;
  int nblocks;         // 32-row blocks to cover (padded total / 32)
};

__global__ void mx_trans_kernel(TransQ a) {
  __shared__ int s_pstart[kMaxExperts + 1];
  const bool padded = a.seg != nullptr;
  if (padded) {
    if (threadIdx.x == 0) {
      int acc = 0;
      for (int e = 0; e < a.nseg; e++) {
        s_pstart[e] = acc;
        const int n = a.seg[e + 1] - a.seg[e];
        acc += (n + kMxSegPad - 1) / kMxSegPad * kMxSegPad;
      }
      s_pstart[a.nseg] = acc;
    }
    __syncthreads();
  }
  const int c = blockIdx.x * blockDim.x + threadIdx.x;  // column
  if (c >= a.cols) return;
  for (int pb = blockIdx.y; pb < a.nblocks; pb += gridDim.y) {
  const int prow = pb * kMxBlock;                       // first padded row of this block
  int e, r0, r1;
  int64_t qb, sb;
  if (padded) {
    if (prow >= s_pstart[a.nseg]) break;
    int lo = 0, hi = a.nseg;  // segment with s_pstart[e] <= prow < s_pstart[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pstart[mid] <= prow) lo = mid; else hi = mid;
    }
    e = lo;
    r0 = a.seg[e] + (prow - s_pstart[e]);
    r1 = a.seg[e + 1];
    qb = (int64_t)c * a.ldq + prow;
    sb = (int64_t)c * a.lds + prow / kMxBlock;
  } else {
    e = prow / a.len;
    const int local = prow - e * a.len;
    r0 = e * a.len + local;
    r1 = (e + 1) * a.len;
    qb = e * a.q_seg + (int64_t)c * a.ldq + a.col_off + local;
    sb = e * a.s_seg + (int64_t)c * a.lds + (a.col_off + local) / kMxBlock;
  }
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const int r = r0 + i;
    v[i] = r < r1 ? bf2f(a.src[(int64_t)r * a.ld_src + c]) : 0.f;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int sexp = mx_scale_exp(amax);
  const float f1 = exp2i(-sexp / 2), f2 = exp2i(-sexp - (-sexp / 2));
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    w[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) w[i] |= e4m3_rne(v[4 * i + j] * f1 * f2) << (8 * j);
  }
  uint4* o = reinterpret_cast<uint4*>(a.q + qb);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  a.s[sb] = (uint8_t)(sexp + 127);
  }
}

}  // namespace

hipError_t mx_quantize_rows(int rows, int cols, const bf16_t* src, uint8_t* q, uint8_t* scales, hipStream_t st) {
  const int64_t n = (int64_t)rows * (cols / kMxBlock);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, rows, cols, src, q, scales);
  return hipGetLastError();
}

static hipError_t launch_trans(TransQ a, int64_t total_rows_pad, hipStream_t st) {
  a.nblocks = (int)((total_rows_pad + kMxBlock - 1) / kMxBlock);
  if (a.cols == 0 || a.nblocks == 0) return hipSuccess;
  const unsigned gy = (unsigned)(a.nblocks < 32768 ? a.nblocks : 32768);
  dim3 grid((unsigned)((a.cols + 255) / 256), gy);
  hipLaunchKernelGGL(mx_trans_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Padded, per-segment transposed quantisation (rows grouped by seg_offsets).
hipError_t mx_quantize_cols_seg(int rows, int cols, const int32_t* seg_offsets, int nseg, const bf16_t* src,
                                uint8_t* q, uint8_t* scales, hipStream_t st) {
  const int rows_pad = rows + kMxSegPad * nseg;
  TransQ a{src, cols, cols, seg_offsets, nseg, 0, q, rows_pad, 0, scales, rows_pad / kMxBlock, 0, 0, 0};
  return launch_trans(a, rows_pad, st);
}


// ---------------------------------------------------------------------------------------
// MXFP8 grouped GEMM: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and one E8M0
// scale per 32 elements along K.  Every operand arrives K-contiguous from the quantisers
// above (activations and forward weights row-wise; weight-gradient operands transposed,
// per expert, 128-padded; backward weights transposed), so the kernel has one operand
// layout.  Operand register layout of the instruction (per lane l, row/column l % 32,
// h = l / 32): bytes 0..15 hold k in [16h, 16h + 16), bytes 16..31 hold k in
// [32 + 16h, 32 + 16h + 16); the lane's scale byte covers the 32-block h of the 64-deep
// step.  Pipeline as in the bf16 kernel: two register stages of bounded buffer loads,
// two swizzled LDS buffers, one barrier per k-step; scale words ride along in registers.
// ---------------------------------------------------------------------------------------
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// fp8 K-contiguous tile [BMN rows][TKB bytes]
template <int BMN, int TKB, int NW>
struct MxOperand {
  static constexpr int TILE_BYTES = BMN * TKB;
  static constexpr int SEGS = TILE_BYTES / 1024;
  static constexpr int ROWS_PER_SEG = 1024 / TKB;
  static constexpr int CPR = TKB / 16;
  static constexpr int PER_THREAD = SEGS / NW;
  static_assert(SEGS % NW == 0, "every wave issues the same number of segments");
  v4i reg[PER_THREAD];

  static __device__ __forceinline__ int swz(int r, int c) {
    if constexpr (CPR == 8) return c ^ ((r >> 1) & 7);
    else return c ^ ((r >> 2) & 3);
  }
  // rows [row0, row_end) valid; columns [k0, k0 + TKB) of each row (live == false: nothing)
  template <class RowPtr>
  __device__ __forceinline__ void load(RowPtr rowptr, int row0, int row_end, int k0, int wave, int lane, bool live) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) {
      const int s = wave + NW * i;
      const int r0 = row0 + s * ROWS_PER_SEG;
      const uint8_t* base = rowptr(r0) + k0;
      const int64_t stride = rowptr(r0 + 1) - rowptr(r0);
      int valid = live ? row_end - r0 : 0;
      valid = valid < 0 ? 0 : (valid > ROWS_PER_SEG ? ROWS_PER_SEG : valid);
      const uint32_t bytes = valid > 0 ? (uint32_t)((valid - 1) * stride + TKB) : 0u;
      const int r = lane / CPR, p = lane % CPR;
      const uint32_t voff = (uint32_t)(r * stride + swz(s * ROWS_PER_SEG + r, p) * 16);
      reg[i] = __builtin_amdgcn_raw_buffer_load_b128(mx_rsrc(base, bytes), voff, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) *reinterpret_cast<v4i*>(lds + (wave + NW * i) * 1024 + lane * 16) = reg[i];
  }
  // operand of 64-deep step s for rows mn0 + lane % 32
  static __device__ __forceinline__ i32x8 frag(const char* lds, int s, int mn0, int lane) {
    const int r = mn0 + (lane & 31), h = lane >> 5;
    const v4i lo = *reinterpret_cast<const v4i*>(lds + r * TKB + (swz(r, 4 * s + h) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + r * TKB + (swz(r, 4 * s + 2 + h) << 4));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

}  // namespace

template <class Cfg, class Prob, int TKB>
__global__ void __launch_bounds__(Cfg::NT) mx_gemm_kernel(const Prob p) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT;
  constexpr int WTM = Cfg::WTM, WTN = Cfg::WTN;
  constexpr int NW = NT / 64;
  using OA = MxOperand<BM, TKB, NW>;
  using OB = MxOperand<BN, TKB, NW>;
  constexpr int STAGE_BYTES = OA::TILE_BYTES + OB::TILE_BYTES;
  __shared__ __attribute__((aligned(1024))) char sm0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sm1[STAGE_BYTES];
  __shared__ int s_map[kMaxExperts + 1];
  __shared__ int s_seg[kMaxExperts + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / Cfg::WAVES_N, wave_n = wave % Cfg::WAVES_N;
  const int E = p.E;
  // group starts: routed rows (Group::M) or 128-padded reduction starts (Group::K)
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e <= E; e++) {
      const int st = p.offsets[e];
      if constexpr (Prob::GROUP == Group::M) {
        s_seg[e] = st;
      } else {
        s_seg[e] = acc;
        if (e < E) acc += (p.offsets[e + 1] - st + kMxSegPad - 1) / kMxSegPad * kMxSegPad;
      }
    }
  }
  __syncthreads();
  auto seg = [&](int e) { return s_seg[e]; };
  const int total_tiles = build_tile_map<Prob::GROUP, BM, BN, NT>(s_map, seg, E, p.M, p.N, tid);
  const int G = gridDim.x;

  for (int t = xcd_logical_wg(); t < total_tiles; t += G) {
    const TileRange tr = tile_at<Prob::GROUP, BM, BN>(t, s_map, seg, E, p.M, p.N, p.K);
    const int e = tr.e, m0 = tr.m0, m_end = tr.m_end, n0 = tr.n0, k_beg = tr.k_beg, k_end = tr.k_end;

    f32x16 acc[WTM][WTN];
#pragma unroll
    for (int i = 0; i < WTM; i++)
#pragma unroll
      for (int j = 0; j < WTN; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    OA ra0, ra1;
    OB rb0, rb1;
    int sa0[WTM], sa1[WTM], sb0[WTN], sb1[WTN];  // scale words (4 blocks) per lane and subtile
    auto load_stage = [&](OA& ra, OB& rb, int (&sa)[WTM], int (&sb)[WTN], int kt) {
      const bool live = kt < k_end;
      ra.load([&](int r) { return p.a_row(e, r); }, m0, m_end, kt, wave, lane, live);
      rb.load([&](int r) { return p.b_row(e, r); }, n0, p.N, kt, wave, lane, live);
      const int word = (kt / kMxBlock) & ~3;  // 4-byte aligned group of block scales
#pragma unroll
      for (int i = 0; i < WTM; i++) {
        const int rb0_ = m0 + (wave_m * WTM + i) * 32;
        int valid = live ? m_end - rb0_ : 0;
        valid = valid < 0 ? 0 : (valid > 32 ? 32 : valid);
        const uint8_t* b0 = p.a_scale_row(e, rb0_);
        const int64_t st = p.a_scale_row(e, rb0_ + 1) - b0;
        sa[i] = __builtin_amdgcn_raw_buffer_load_b32(mx_rsrc(b0, valid > 0 ? (uint32_t)(valid * st) : 0u),
                                                     (uint32_t)((lane & 31) * st + word), 0, 0);
      }
#pragma unroll
      for (int j = 0; j < WTN; j++) {
        const int nb0 = n0 + (wave_n * WTN + j) * 32;
        int valid = live ? p.N - nb0 : 0;
        valid = valid < 0 ? 0 : (valid > 32 ? 32 : valid);
        const uint8_t* b0 = p.b_scale_row(e, nb0);
        const int64_t st = p.b_scale_row(e, nb0 + 1) - b0;
        sb[j] = __builtin_amdgcn_raw_buffer_load_b32(mx_rsrc(b0, valid > 0 ? (uint32_t)(valid * st) : 0u),
                                                     (uint32_t)((lane & 31) * st + word), 0, 0);
      }
    };
    auto store_stage = [&](const OA& ra, const OB& rb, char* base) {
      ra.store(base, wave, lane);
      rb.store(base + OA::TILE_BYTES, wave, lane);
    };
    auto compute = [&](const char* st, const int (&sa)[WTM], const int (&sb)[WTN], int kt) {
      const int byte0 = (kt / kMxBlock) & 3;
#pragma unroll
      for (int s = 0; s < TKB / 64; s++) {
        i32x8 af[WTM], bfr[WTN];
        int xa[WTM], xb[WTN];
        const int sh = 8 * (byte0 + 2 * s + (lane >> 5));
#pragma unroll
        for (int i = 0; i < WTM; i++) {
          af[i] = OA::frag(st, s, (wave_m * WTM + i) * 32, lane);
          xa[i] = (sa[i] >> sh) & 0xff;
        }
#pragma unroll
        for (int j = 0; j < WTN; j++) {
          bfr[j] = OB::frag(st + OA::TILE_BYTES, s, (wave_n * WTN + j) * 32, lane);
          xb[j] = (sb[j] >> sh) & 0xff;
        }
#pragma unroll
        for (int i = 0; i < WTM; i++)
#pragma unroll
          for (int j = 0; j < WTN; j++)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0, xa[i], 0,
                                                                         xb[j]);
      }
    };
    auto lds_barrier = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    const int nk = (k_end - k_beg + TKB - 1) / TKB;
    if (nk > 0) {
      load_stage(ra0, rb0, sa0, sb0, k_beg);
      load_stage(ra1, rb1, sa1, sb1, k_beg + TKB);
      lds_barrier();
      store_stage(ra0, rb0, sm0);
      int cs0[WTM], cs0b[WTN];  // scales of the stage now in sm0
#pragma unroll
      for (int i = 0; i < WTM; i++) cs0[i] = sa0[i];
#pragma unroll
      for (int j = 0; j < WTN; j++) cs0b[j] = sb0[j];
      load_stage(ra0, rb0, sa0, sb0, k_beg + 2 * TKB);
      lds_barrier();
      int cs1[WTM], cs1b[WTN];
      for (int it = 0; it < nk; it += 2) {
        compute(sm0, cs0, cs0b, k_beg + it * TKB);
        if (it + 1 < nk) store_stage(ra1, rb1, sm1);
#pragma unroll
        for (int i = 0; i < WTM; i++) cs1[i] = sa1[i];
#pragma unroll
        for (int j = 0; j < WTN; j++) cs1b[j] = sb1[j];
        load_stage(ra1, rb1, sa1, sb1, k_beg + (it + 3) * TKB);
        lds_barrier();
        if (it + 1 < nk) compute(sm1, cs1, cs1b, k_beg + (it + 1) * TKB);
        if (it + 2 < nk) store_stage(ra0, rb0, sm0);
#pragma unroll
        for (int i = 0; i < WTM; i++) cs0[i] = sa0[i];
#pragma unroll
        for (int j = 0; j < WTN; j++) cs0b[j] = sb0[j];
        load_stage(ra0, rb0, sa0, sb0, k_beg + (it + 4) * TKB);
        lds_barrier();
      }
    }

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
            if (hcol < p.N / 2) p.epilogue_swiglu(m, hcol, acc[i][j][r], acc[i][j + 1][r]);
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
// Problems.  Codes q* [rows][K] and scales s* [rows][K/32] (K-contiguous).
// ---------------------------------------------------------------------------------------
struct MxBase {
  int M = 0, N = 0, K = 0, E = 1;
  const int* offsets = nullptr;
  const uint8_t *qa = nullptr, *sa = nullptr;  // A codes / scales, row length K (padded for Group::K)
  int64_t lda = 0;                             // bytes per A row (= K)
};

struct MxGemm1 : MxBase {  // [a | b] = X [W1 | W3]^T, SwiGLU epilogue
  static constexpr Group GROUP = Group::M;
  static constexpr Epi EPI = Epi::SwiGLU;
  int f = 0;
  const uint8_t *q1 = nullptr, *s1 = nullptr, *q3 = nullptr, *s3 = nullptr;  // [E][f][d]
  bf16_t *ab = nullptr, *h = nullptr;
  __device__ const uint8_t* a_row(int, int m) const { return qa + (int64_t)m * K; }
  __device__ const uint8_t* a_scale_row(int, int m) const { return sa + (int64_t)m * (K / kMxBlock); }
  __device__ int64_t brow(int e, int n) const { return (int64_t)e * f + ((n >> 5) >> 1) * 32 + (n & 31); }
  __device__ const uint8_t* b_row(int e, int n) const { return ((n >> 5) & 1 ? q3 : q1) + brow(e, n) * K; }
  __device__ const uint8_t* b_scale_row(int e, int n) const {
    return ((n >> 5) & 1 ? s3 : s1) + brow(e, n) * (K / kMxBlock);
  }
  __device__ void epilogue_swiglu(int m, int hcol, float a, float b) const {
    bf16_t* abr = ab + (int64_t)m * 2 * f;
    abr[hcol] = f2bf(a);
    abr[f + hcol] = f2bf(b);
    h[(int64_t)m * f + hcol] = f2bf(a * sigmoidf_(a) * b);
  }
  __device__ void epilogue(int, int, int, float) const {}
};

struct MxPlain : MxBase {  // C[m][n] = sum_k A[m][k] B_e[n][k], bf16 out (Group::M)
  static constexpr Group GROUP = Group::M;
  static constexpr Epi EPI = Epi::Store;
  const uint8_t *qb = nullptr, *sb = nullptr;  // [E][N][K]
  bf16_t* C = nullptr;
  __device__ const uint8_t* a_row(int, int m) const { return qa + (int64_t)m * K; }
  __device__ const uint8_t* a_scale_row(int, int m) const { return sa + (int64_t)m * (K / kMxBlock); }
  __device__ const uint8_t* b_row(int e, int n) const { return qb + ((int64_t)e * N + n) * K; }
  __device__ const uint8_t* b_scale_row(int e, int n) const { return sb + ((int64_t)e * N + n) * (K / kMxBlock); }
  __device__ void epilogue(int, int m, int n, float v) const { C[(int64_t)m * N + n] = f2bf(v); }
};

struct MxDgrad2 : MxPlain {  // dh = dy W2_e, then the SwiGLU gradient from the saved a, b
  static constexpr Epi EPI = Epi::DSwiGLU;
  const bf16_t* ab = nullptr;
  bf16_t* dab = nullptr;
  __device__ void epilogue(int, int m, int n, float dh) const {
    const bf16_t* abr = ab + (int64_t)m * 2 * N;
    const float a = bf2f(abr[n]), b = bf2f(abr[N + n]);
    const float s = sigmoidf_(a);
    bf16_t* o = dab + (int64_t)m * 2 * N;
    o[n] = f2bf(dh * b * s * (1.f + a * (1.f - s)));
    o[N + n] = f2bf(dh * a * s);
  }
};

struct MxWgrad : MxBase {  // C_e[m][n] = sum over expert e's (padded) rows of A^T B (Group::K)
  static constexpr Group GROUP = Group::K;
  static constexpr Epi EPI = Epi::Store;
  const uint8_t *qb = nullptr, *sb = nullptr;  // [N][Kpad]
  bf16_t* C0 = nullptr;  // rows m < split
  bf16_t* C1 = nullptr;  // rows m >= split (may be null)
  int split = 0;
  __device__ const uint8_t* a_row(int, int m) const { return qa + (int64_t)m * K; }
  __device__ const uint8_t* a_scale_row(int, int m) const { return sa + (int64_t)m * (K / kMxBlock); }
  __device__ const uint8_t* b_row(int, int n) const { return qb + (int64_t)n * K; }
  __device__ const uint8_t* b_scale_row(int, int n) const { return sb + (int64_t)n * (K / kMxBlock); }
  __device__ void epilogue(int e, int m, int n, float v) const {
    bf16_t* W = m < split ? C0 + ((int64_t)e * split + m) * N : C1 + ((int64_t)e * (M - split) + (m - split)) * N;
    W[n] = f2bf(v);
  }
};

template <class Prob>
static hipError_t launch_mx(const Prob& p, hipStream_t st) {
  using Cfg = TileCfg<128, 256, 2, 4>;
  const auto kern = mx_gemm_kernel<Cfg, Prob, 128>;
  static int occ = 0;
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, Cfg::NT, 0) != hipSuccess || o < 1) o = 1;
    occ = o;
  }
  int64_t bound;
  const int64_t ntn = (p.N + Cfg::BN - 1) / Cfg::BN;
  if constexpr (Prob::GROUP == Group::M) bound = ((int64_t)p.M / Cfg::BM + p.E) * ntn;
  else bound = (int64_t)p.E * ((p.M + Cfg::BM - 1) / Cfg::BM) * ntn;
  int64_t G = (int64_t)device_cu_count() * occ;
  if (bound < G) G = bound;
  G = ((G + 7) / 8) * 8;
  if (G < 8) G = 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(Cfg::NT), 0, st, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Workspace: each GEMM call quantises its two operands into [A codes | A scales | B codes |
// B scales] at the start of ws (regions 256-byte aligned); calls on one workspace must be
// ordered on the stream.
// ---------------------------------------------------------------------------------------
static size_t al(size_t b) { return (b + 255) / 256 * 256; }
static size_t qbytes(int64_t rows, int64_t K) { return al((size_t)(rows * K)) + al((size_t)(rows * (K / kMxBlock))); }

size_t mx_workspace_bytes(int R, int d, int f, int E) {
  const int64_t Rp = (int64_t)R + (int64_t)kMxSegPad * E;
  size_t m = 0;
  auto upd = [&](size_t v) { m = v > m ? v : m; };
  upd(qbytes(R, d) + 2 * qbytes((int64_t)E * f, d));   // gemm1
  upd(qbytes(R, f) + qbytes((int64_t)E * d, f));       // gemm2
  upd(qbytes(R, d) + qbytes((int64_t)E * f, d));       // dgrad2
  upd(qbytes(R, 2 * f) + qbytes((int64_t)E * d, 2 * f));  // dgrad1
  upd(qbytes(d, Rp) + qbytes(f, Rp));                  // wgrad2
  upd(qbytes(2 * f, Rp) + qbytes(d, Rp));              // wgrad1
  return m;
}

namespace {
struct Carve {
  char* p;
  uint8_t* take(size_t b) {
    uint8_t* r = reinterpret_cast<uint8_t*>(p);
    p += al(b);
    return r;
  }
};
}  // namespace

hipError_t gemm1_fwd_mx(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* W1, const bf16_t* W3,
                        bf16_t* ab, bf16_t* h, void* ws, hipStream_t st) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ef = (int64_t)s.E * s.f;
  uint8_t *xq = c.take((size_t)s.R * s.d), *xs = c.take((size_t)s.R * s.d / kMxBlock);
  uint8_t *q1 = c.take((size_t)Ef * s.d), *s1 = c.take((size_t)Ef * s.d / kMxBlock);
  uint8_t *q3 = c.take((size_t)Ef * s.d), *s3 = c.take((size_t)Ef * s.d / kMxBlock);
  hipError_t err;
  if ((err = mx_quantize_rows(s.R, s.d, X, xq, xs, st)) != hipSuccess) return err;
  if ((err = mx_quantize_rows((int)Ef, s.d, W1, q1, s1, st)) != hipSuccess) return err;
  if ((err = mx_quantize_rows((int)Ef, s.d, W3, q3, s3, st)) != hipSuccess) return err;
  MxGemm1 p;
  p.M = s.R; p.N = 2 * s.f; p.K = s.d; p.E = s.E; p.offsets = offsets; p.qa = xq; p.sa = xs; p.f = s.f;
  p.q1 = q1; p.s1 = s1; p.q3 = q3; p.s3 = s3; p.ab = ab; p.h = h;
  return launch_mx(p, st);
}

hipError_t gemm2_fwd_mx(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* W2, bf16_t* Y,
                        void* ws, hipStream_t st) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ed = (int64_t)s.E * s.d;
  uint8_t *hq = c.take((size_t)s.R * s.f), *hs = c.take((size_t)s.R * s.f / kMxBlock);
  uint8_t *wq = c.take((size_t)Ed * s.f), *wsc = c.take((size_t)Ed * s.f / kMxBlock);
  hipError_t err;
  if ((err = mx_quantize_rows(s.R, s.f, H, hq, hs, st)) != hipSuccess) return err;
  if ((err = mx_quantize_rows((int)Ed, s.f, W2, wq, wsc, st)) != hipSuccess) return err;
  MxPlain p;
  p.M = s.R; p.N = s.d; p.K = s.f; p.E = s.E; p.offsets = offsets; p.qa = hq; p.sa = hs;
  p.qb = wq; p.sb = wsc; p.C = Y;
  return launch_mx(p, st);
}

// Transposed per-expert weight quantisation: W_e [rows_e][cols] -> [cols][k_len] blocks
// along rows_e, written at column offset col_off of each output row.
static hipError_t quantize_weight_t(int E, int rows_e, int cols, const bf16_t* W, uint8_t* q, uint8_t* sc,
                                    int k_len, int col_off, hipStream_t st) {
  TransQ a{W, cols, cols, nullptr, E, rows_e, q, k_len, (int64_t)cols * k_len, sc, k_len / kMxBlock,
           (int64_t)cols * (k_len / kMxBlock), col_off, 0};
  return launch_trans(a, (int64_t)E * rows_e, st);
}

hipError_t dgrad2_mx(const GemmShape& s, const int* offsets, const bf16_t* dY, const bf16_t* W2, const bf16_t* ab,
                     bf16_t* dab, void* ws, hipStream_t st) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ef = (int64_t)s.E * s.f;
  uint8_t *yq = c.take((size_t)s.R * s.d), *ys = c.take((size_t)s.R * s.d / kMxBlock);
  uint8_t *wq = c.take((size_t)Ef * s.d), *wsc = c.take((size_t)Ef * s.d / kMxBlock);
  hipError_t err;
  if ((err = mx_quantize_rows(s.R, s.d, dY, yq, ys, st)) != hipSuccess) return err;
  if ((err = quantize_weight_t(s.E, s.d, s.f, W2, wq, wsc, s.d, 0, st)) != hipSuccess) return err;  // W2_e^T [f][d]
  MxDgrad2 p;
  p.M = s.R; p.N = s.f; p.K = s.d; p.E = s.E; p.offsets = offsets; p.qa = yq; p.sa = ys;
  p.qb = wq; p.sb = wsc; p.ab = ab; p.dab = dab;
  return launch_mx(p, st);
}

hipError_t dgrad1_mx(const GemmShape& s, const int* offsets, const bf16_t* dab, const bf16_t* W1, const bf16_t* W3,
                     bf16_t* dX, void* ws, hipStream_t st) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ed = (int64_t)s.E * s.d;
  uint8_t *gq = c.take((size_t)s.R * 2 * s.f), *gs = c.take((size_t)s.R * 2 * s.f / kMxBlock);
  uint8_t *wq = c.take((size_t)Ed * 2 * s.f), *wsc = c.take((size_t)Ed * 2 * s.f / kMxBlock);
  hipError_t err;
  if ((err = mx_quantize_rows(s.R, 2 * s.f, dab, gq, gs, st)) != hipSuccess) return err;
  // [W1_e ; W3_e]^T = [d][2f]: W1_e^T in columns [0, f), W3_e^T in [f, 2f)
  if ((err = quantize_weight_t(s.E, s.f, s.d, W1, wq, wsc, 2 * s.f, 0, st)) != hipSuccess) return err;
  if ((err = quantize_weight_t(s.E, s.f, s.d, W3, wq, wsc, 2 * s.f, s.f, st)) != hipSuccess) return err;
  MxPlain p;
  p.M = s.R; p.N = s.d; p.K = 2 * s.f; p.E = s.E; p.offsets = offsets; p.qa = gq; p.sa = gs;
  p.qb = wq; p.sb = wsc; p.C = dX;
  return launch_mx(p, st);
}

hipError_t wgrad2_mx(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* dY, bf16_t* dW2,
                     void* ws, hipStream_t st) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Rp = (int64_t)s.R + (int64_t)kMxSegPad * s.E;
  uint8_t *aq = c.take((size_t)(s.d * Rp)), *as = c.take((size_t)(s.d * Rp / kMxBlock));
  uint8_t *bq = c.take((size_t)(s.f * Rp)), *bs = c.take((size_t)(s.f * Rp / kMxBlock));
  hipError_t err;
  if ((err = mx_quantize_cols_seg(s.R, s.d, offsets, s.E, dY, aq, as, st)) != hipSuccess) return err;
  if ((err = mx_quantize_cols_seg(s.R, s.f, offsets, s.E, H, bq, bs, st)) != hipSuccess) return err;
  MxWgrad p;
  p.M = s.d; p.N = s.f; p.K = (int)Rp; p.E = s.E; p.offsets = offsets; p.qa = aq; p.sa = as;
  p.qb = bq; p.sb = bs; p.C0 = dW2; p.split = s.d;
  return launch_mx(p, st);
}

hipError_t wgrad1_mx(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* dab, bf16_t* dW1,
                     bf16_t* dW3, void* ws, hipStream_t st) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Rp = (int64_t)s.R + (int64_t)kMxSegPad * s.E;
  uint8_t *aq = c.take((size_t)(2 * s.f * Rp)), *as = c.take((size_t)(2 * s.f * Rp / kMxBlock));
  uint8_t *bq = c.take((size_t)(s.d * Rp)), *bs = c.take((size_t)(s.d * Rp / kMxBlock));
  hipError_t err;
  if ((err = mx_quantize_cols_seg(s.R, 2 * s.f, offsets, s.E, dab, aq, as, st)) != hipSuccess) return err;
  if ((err = mx_quantize_cols_seg(s.R, s.d, offsets, s.E, X, bq, bs, st)) != hipSuccess) return err;
  MxWgrad p;
  p.M = 2 * s.f; p.N = s.d; p.K = (int)Rp; p.E = s.E; p.offsets = offsets; p.qa = aq; p.sa = as;
  p.qb = bq; p.sb = bs; p.C0 = dW1; p.C1 = dW3; p.split = s.f;
  return launch_mx(p, st);
}

}  // namespace moe
