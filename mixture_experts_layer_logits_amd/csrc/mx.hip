// MXFP8 block quantisation on the device: bf16 -> E4M3 codes + one E8M0 scale per 32
// elements.  MXFP8 is the reduced-precision format the pages report for the expert FFN
// compute and expert data movement (unite.ai, "Ai2 κυκλοφορεί το Olmo-Core 3…",
// section "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"; ettayeb.fr, "Olmo-core 3
// ouvre l'entraînement des MoE…", section "Trois parallélismes, trois optimisations de
// routage").
//
// Scale: the smallest 2^s with amax * 2^-s <= 448 (E4M3's largest finite value),
// s clamped to [-127, 127]; blocks whose amax is zero or an fp32 subnormal get -127.
// Elements: v * 2^-s (exact in fp32) rounded to nearest-even onto the E4M3 grid by
// gfx950's packed fp8 conversion, two elements per instruction; a GPU test checks it
// against the oracle's encoder on every bf16 value of magnitude <= 448.
#include <cstdlib>
#include <cstring>

#include "common.h"
#include "mx.h"
#include "mxcode.h"
#include "tilemap.h"
#include "epilogue.h"

namespace moe {

namespace {

// one thread per 32-element block of a row.  il_rows > 0: the rows are E stacked weights
// of il_rows rows each, written to the 32-row-interleaved pair layout of the forward GEMM
// (block b of weight e lands at rows e * 2 il_rows + 64 (b / 32) + 32 il_which + b % 32).
__global__ void mx_rows_kernel(int rows, int cols, const bf16_t* __restrict__ src, uint8_t* __restrict__ q,
                               uint8_t* __restrict__ scales, int il_rows, int il_which) {
  const int nb = cols / kMxBlock;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= (int64_t)rows * nb) return;
  const bf16_t* p = src + b * kMxBlock;
  int64_t ob = b;
  if (il_rows > 0) {
    const int64_t row = b / nb, e = row / il_rows, rr = row % il_rows;
    const int64_t orow = e * 2 * il_rows + ((rr >> 5) << 6) + ((int64_t)il_which << 5) + (rr & 31);
    ob = orow * nb + b % nb;
  }
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
  const float r = mx_inv_scale(s);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; i++) w[i] = e4m3x4(v[4 * i] * r, v[4 * i + 1] * r, v[4 * i + 2] * r, v[4 * i + 3] * r);
  uint4* o = reinterpret_cast<uint4*>(q + ob * kMxBlock);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[ob] = (uint8_t)(s + 127);
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
};

// One workgroup per tile of 128 source rows (four 32-row blocks of one segment; output
// segments are padded to 128 rows, so a tile never straddles two) by 64 columns.  Rows
// are read as 16-byte chunks into LDS, each thread then quantises one 32-row block of one
// column, and the codes leave through a second LDS tile as full 128-byte lines of the
// transposed output.
constexpr int kTransRows = 128, kTransCols = 64, kTransThreads = 256;
constexpr int kTransOutPitch = kTransRows + 16;  // bytes per staged output row (bank spread)

__global__ void __launch_bounds__(kTransThreads) mx_trans_kernel(TransQ a) {
  __shared__ int s_pstart[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) bf16_t s_in[kTransRows][kTransCols];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[kTransCols][kTransOutPitch];
  __shared__ uint32_t s_csc[kTransCols];  // the tile's four 32-row block scales of each column
  const int tid = threadIdx.x;
  const bool padded = a.seg != nullptr;
  if (padded) {
    if (tid == 0) {
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
  const int c0 = blockIdx.x * kTransCols;
  const int tiles_per_seg = (a.len + kTransRows - 1) / kTransRows;  // uniform mode
  const int ntiles = padded ? s_pstart[a.nseg] / kTransRows : a.nseg * tiles_per_seg;
  for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
    // source rows [r0, r1) of segment e; output rows start at local row `lrow` of the
    // segment's output, nblk 32-row blocks are stored
    int r0, r1, nblk;
    int64_t qrow0, srow0;  // output offsets of (column 0, local row lrow)
    if (padded) {
      const int prow = tile * kTransRows;
      int lo = 0, hi = a.nseg;  // segment with s_pstart[e] <= prow < s_pstart[e+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pstart[mid] <= prow) lo = mid; else hi = mid;
      }
      r0 = a.seg[lo] + (prow - s_pstart[lo]);
      r1 = a.seg[lo + 1];
      nblk = 4;
      qrow0 = prow;
      srow0 = prow / kMxBlock;
    } else {
      const int e = tile / tiles_per_seg, local = (tile % tiles_per_seg) * kTransRows;
      r0 = e * a.len + local;
      r1 = (e + 1) * a.len;
      nblk = (a.len - local) / kMxBlock < 4 ? (a.len - local) / kMxBlock : 4;
      qrow0 = e * a.q_seg + a.col_off + local;
      srow0 = e * a.s_seg + (a.col_off + local) / kMxBlock;
    }
    // 128 rows x 128 bytes in 16-byte chunks, rows past the segment read as zero
#pragma unroll
    for (int i = 0; i < kTransRows * kTransCols * 2 / 16 / kTransThreads; i++) {
      const int q = tid + kTransThreads * i, row = q >> 3, ch = q & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r0 + row < r1 && c0 + ch * 8 < a.cols)  // columns come in whole 8-column chunks (cols % 32 == 0)
        v = *reinterpret_cast<const uint4*>(a.src + (int64_t)(r0 + row) * a.ld_src + c0 + ch * 8);
      *reinterpret_cast<uint4*>(&s_in[row][ch * 8]) = v;
    }
    __syncthreads();
    {
      const int c = tid & (kTransCols - 1), b = tid >> 6;  // column, 32-row block (one per wave)
      float v[32];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        v[i] = bf2f(s_in[b * 32 + i][c]);
        amax = fmaxf(amax, fabsf(v[i]));
      }
      const int sexp = mx_scale_exp(amax);
      const float r = mx_inv_scale(sexp);
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; i++) w[i] = e4m3x4(v[4 * i] * r, v[4 * i + 1] * r, v[4 * i + 2] * r, v[4 * i + 3] * r);
      uint4* o = reinterpret_cast<uint4*>(&s_out[c][b * 32]);
      o[0] = make_uint4(w[0], w[1], w[2], w[3]);
      o[1] = make_uint4(w[4], w[5], w[6], w[7]);
      reinterpret_cast<uint8_t*>(s_csc)[c * 4 + b] = (uint8_t)(sexp + 127);
    }
    __syncthreads();
    // the scales of column c0 + c are nblk consecutive bytes: one 4-byte store per column
    // when all four blocks are stored and the word is aligned, else byte by byte
    if (tid < kTransCols && c0 + tid < a.cols) {
      uint8_t* dst = a.s + srow0 + (int64_t)(c0 + tid) * a.lds;
      const uint32_t w = s_csc[tid];
      if (nblk == 4 && (reinterpret_cast<uintptr_t>(dst) & 3) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = w;
      } else {
        for (int b = 0; b < nblk; b++) dst[b] = (uint8_t)(w >> (8 * b));
      }
    }
    // 64 output rows x (32 * nblk) bytes, 8 lanes per 128-byte row
#pragma unroll
    for (int i = 0; i < kTransCols * kTransRows / 16 / kTransThreads; i++) {
      const int q = tid + kTransThreads * i, c = q >> 3, ch = q & 7;
      if (ch * 16 < nblk * kMxBlock && c0 + c < a.cols)
        *reinterpret_cast<uint4*>(a.q + qrow0 + (int64_t)(c0 + c) * a.ldq + ch * 16) =
            *reinterpret_cast<const uint4*>(&s_out[c][ch * 16]);
    }
    __syncthreads();  // s_in / s_out are reused by the next tile
  }
}

// ---------------------------------------------------------------------------------------
// MXFP8 dispatch: the routed rows v_r, r in [0, R), are gathered from their tokens and
// leave only as block-quantised codes, in both layouts the expert GEMMs read, so no bf16
// copy of them is ever written (MXFP8 for the data moved to the experts: unite.ai, section
// "Παραλληλισμός, Ακρίβεια και Τεχνικές Μνήμης"):
//   row layout     q_rows [R][cols], s_rows [R][cols / 32]        (as mx_quantize_rows)
//   column layout  q_cols [cols][ld], s_cols [cols][ld / 32]       (as mx_quantize_cols_seg:
//                  blocks down each column restarting at every expert, experts padded to
//                  128 rows at P_e = sum_{e'<e} roundup(n_e', 128))
// v_r = src[row_src[r]], or with gates v_r = bf16(gates[t, j] * src[t]) for r = slot_row[t, j]
// (the product rounded once to bf16, as the routed output gradient is stored in bf16).
//
// A workgroup owns one 128-row tile of the padded row space (rows of one expert: its token
// ids and gates are looked up once) and a run of 64-column tiles.  Per column tile each
// thread loads four 16-byte chunks (consecutive lanes on consecutive chunks of a row; the
// next tile's chunks are in flight while the current one is worked on), quantises its row
// blocks in registers (a 32-column block spans the four lanes of a quad), and stages the
// bf16 values in LDS; each lane then quantises one column's 32-row block from LDS, and the
// codes leave through an LDS tile as full 128-byte lines of the column layout.  The row
// layout gets 64-byte halves of its lines from consecutive column tiles of one workgroup.
// The kernel is bound by its vector-memory instruction count, so its stores are few and
// wide: row codes leave 16 bytes per lane (lane pairs swap one row's 8 codes), each lane
// stores at most one row-scale pair, and one wave stores a tile's four column-scale bytes
// of each column as one word.
// ---------------------------------------------------------------------------------------
struct DispatchQ {
  const bf16_t* src;  // [T][cols]
  int cols;
  const int32_t* row_src;  // [R]
  const int32_t* seg;      // expert offsets [nseg + 1]
  int nseg;
  const float* gates;       // [T][k], nullptr: ungated
  const int32_t* slot_row;  // [T][k] (gated only)
  int k;
  uint8_t* q_rows;
  uint8_t* s_rows;
  uint8_t* q_cols;
  uint8_t* s_cols;
  int64_t ld;     // row count of the column layout (R + 128 nseg)
  int col_tiles;  // column tiles per workgroup
};

constexpr int kDispRows = 128, kDispCols = 64, kDispThreads = 256;
constexpr int kDispRowChunks = kDispCols * 2 / 16;             // 16-byte chunks per staged row: 8
constexpr int kDispInPitch = kDispCols * 2 + 16;               // bytes per staged bf16 row (bank spread)
constexpr int kDispOutPitch = kDispRows + 16;                  // bytes per staged column of codes
constexpr int kDispChunks = kDispRows * kDispRowChunks / kDispThreads;  // chunks per thread: 4
constexpr int kDispRowStep = kDispThreads / kDispRowChunks;    // rows between a thread's chunks: 32
static_assert(kDispCols * kDispOutPitch <= kDispRows * kDispInPitch, "code tile reuses the input tile");
static_assert((kMaxExperts + 1) * 4 <= kDispRows * kDispInPitch, "segment scan reuses the input tile");
static_assert(kDispCols == kWave && kDispRows == 32 * (kDispThreads / kWave), "one column per lane, one block per wave");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float quad_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false)));
}

__device__ __forceinline__ void widen_bf16x8(const uint4& q, float (&v)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__global__ void __launch_bounds__(kDispThreads) mx_dispatch_kernel(DispatchQ a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kDispRows * kDispInPitch];
  __shared__ int s_tok[kDispRows];
  __shared__ float s_gate[kDispRows];
  __shared__ int s_wsum[kDispThreads / kWave];
  __shared__ uint32_t s_csc[kDispCols];  // the tile's column scale bytes, 4 per column
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  // --- padded tile starts of the experts (exclusive scan of roundup(n_e, 128) / 128),
  //     four experts per thread, in s_buf; then the expert owning this row tile
  int* s_tstart = reinterpret_cast<int*>(s_buf);
  {
    int cnt[4], local = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int e = tid * 4 + u;
      cnt[u] = e < a.nseg ? (a.seg[e + 1] - a.seg[e] + kDispRows - 1) / kDispRows : 0;
      local += cnt[u];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int excl = incl - local;
    for (int w = 0; w < wave; w++) excl += s_wsum[w];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int e = tid * 4 + u;
      if (e < a.nseg) s_tstart[e] = excl;
      excl += cnt[u];
    }
    if (tid == 0) s_tstart[a.nseg] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
  }
  const int rt = blockIdx.x;
  if (rt >= s_tstart[a.nseg]) return;  // whole workgroup: past the last padded tile
  int e = 0;
  {
    int hi = a.nseg;  // last expert with s_tstart[e] <= rt (it owns >= 1 tile)
    while (hi - e > 1) {
      const int mid = (e + hi) >> 1;
      if (s_tstart[mid] <= rt) e = mid; else hi = mid;
    }
  }
  const int r0 = a.seg[e] + (rt - s_tstart[e]) * kDispRows;
  const int nvalid = min(kDispRows, a.seg[e + 1] - r0);
  const int64_t prow = (int64_t)rt * kDispRows;  // first row of this tile in the column layout
  if (tid < kDispRows) {
    int t = -1;
    float g = 1.f;
    if (tid < nvalid) {
      const int r = r0 + tid;
      t = a.row_src[r];
      if (a.gates) {
        for (int j = 0; j < a.k; j++)
          if (a.slot_row[(int64_t)t * a.k + j] == r) g = a.gates[(int64_t)t * a.k + j];
      }
    }
    s_tok[tid] = t;
    s_gate[tid] = g;
  }
  __syncthreads();  // s_tstart is dead from here on; s_buf becomes the tile buffer

  const int chunk = tid % kDispRowChunks, row_base = tid / kDispRowChunks;  // rows row_base + 32 i
  const int ct_begin = blockIdx.y * a.col_tiles;
  const int ct_end = min(ct_begin + a.col_tiles, a.cols / kDispCols);
  const int nbc = a.cols / kMxBlock;
  // a thread's source rows (padding rows read row 0 and are zeroed after the load, so no
  // load sits in a branch)
  const bf16_t* srcp[kDispChunks];
  uint32_t keep[kDispChunks];  // all ones for a routed row, zero for padding
#pragma unroll
  for (int i = 0; i < kDispChunks; i++) {
    const int t = s_tok[row_base + kDispRowStep * i];
    keep[i] = t >= 0 ? 0xffffffffu : 0u;
    srcp[i] = a.src + (int64_t)(t < 0 ? 0 : t) * a.cols + chunk * 8;
  }
  // the row layout of this tile's rows as one buffer: stores of padding rows fall past its
  // end and are dropped by the hardware, so no store sits in a branch either
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(a.q_rows + (int64_t)r0 * a.cols, (short)0, nvalid * a.cols, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(a.s_rows + (int64_t)r0 * nbc, (short)0, nvalid * nbc, 0x00020000);

  auto load = [&](uint4 (&v)[kDispChunks], int ct) {
#pragma unroll
    for (int i = 0; i < kDispChunks; i++) v[i] = *reinterpret_cast<const uint4*>(srcp[i] + ct * kDispCols);
  };
  uint4 cur[kDispChunks], nxt[kDispChunks];
  if (ct_begin < ct_end) load(cur, ct_begin);
  for (int ct = ct_begin; ct < ct_end; ct++) {
    const int c0 = ct * kDispCols;
    load(nxt, min(ct + 1, ct_end - 1));  // the next tile's rows are in flight during this one
    // --- row blocks, straight from registers
    uint2 codes[kDispChunks];
    uint32_t sw[kDispChunks];
#pragma unroll
    for (int i = 0; i < kDispChunks; i++) {
      const int row = row_base + kDispRowStep * i;
      cur[i] = make_uint4(cur[i].x & keep[i], cur[i].y & keep[i], cur[i].z & keep[i], cur[i].w & keep[i]);
      float v[8];
      widen_bf16x8(cur[i], v);
      if (a.gates) {  // v = bf16(g * src): the stored routed gradient
        const float g = s_gate[row];
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; u++) w[u] = (uint32_t)f2bf(g * v[2 * u]) | ((uint32_t)f2bf(g * v[2 * u + 1]) << 16);
        cur[i] = make_uint4(w[0], w[1], w[2], w[3]);
        widen_bf16x8(cur[i], v);
      }
      float amax = 0.f;
#pragma unroll
      for (int u = 0; u < 8; u++) amax = fmaxf(amax, fabsf(v[u]));
      amax = quad_max<0xB1>(amax);  // the four lanes of a 32-column block
      amax = quad_max<0x4E>(amax);
      const int sexp = mx_scale_exp(amax);
      const float r = mx_inv_scale(sexp);
      const uint32_t w0 = e4m3x4(v[0] * r, v[1] * r, v[2] * r, v[3] * r);
      const uint32_t w1 = e4m3x4(v[4] * r, v[5] * r, v[6] * r, v[7] * r);
      // the scale bytes of the row's two blocks, gathered into the lane of chunk 0
      const uint32_t sb = (uint32_t)(sexp + 127);
      sw[i] = sb | (__shfl_down(sb, 4, kDispRowChunks) << 8);
      codes[i] = make_uint2(w0, w1);
      *reinterpret_cast<uint4*>(s_buf + row * kDispInPitch + chunk * 16) = cur[i];
    }
    // row codes as 16-byte stores: the lanes of chunks 2c and 2c + 1 (lane ^ 1) pair up, the
    // even one storing both chunks of row i, the odd one of row i + 1 (i = 0, 2)
    {
      const bool odd = chunk & 1;
#pragma unroll
      for (int i = 0; i < kDispChunks; i += 2) {
        const uint2 give = odd ? codes[i] : codes[i + 1];  // the partner's row
        const uint32_t g0 = __shfl_xor(give.x, 1, kWave), g1 = __shfl_xor(give.y, 1, kWave);
        const int row = row_base + kDispRowStep * (i + (odd ? 1 : 0));
        const u32x4 v = odd ? u32x4{g0, g1, codes[i + 1].x, codes[i + 1].y} : u32x4{codes[i].x, codes[i].y, g0, g1};
        __builtin_amdgcn_raw_buffer_store_b128(v, rq, row * a.cols + c0 + (chunk & ~1) * 8, 0, 0);
      }
    }
    // row scales, one store per lane: the lane of chunk c < 4 stores the two scale bytes of
    // row row_base + 32 c (held by the chunk-0 lane of its row group); the other lanes'
    // stores are aimed past the buffer and dropped
    {
      uint32_t mine = 0;
#pragma unroll
      for (int i = 0; i < kDispChunks; i++) {
        const uint32_t v = __shfl(sw[i], lane & ~(kDispRowChunks - 1), kWave);
        if (chunk == i) mine = v;
      }
      __builtin_amdgcn_raw_buffer_store_b16(
          (uint16_t)mine, rs, chunk < kDispChunks ? (row_base + kDispRowStep * chunk) * nbc + c0 / kMxBlock : 0x7ffffff0,
          0, 0);
    }
    __syncthreads();
    // --- column blocks: wave w takes rows [32 w, 32 w + 32) of column `lane`; two passes
    //     over the staged values (block maximum, then the codes)
    uint32_t q[8];
    {
      const uint8_t* col = s_buf + wave * 32 * kDispInPitch + lane * 2;
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 32; i++)
        m = fmaxf(m, fabsf(bf2f(*reinterpret_cast<const bf16_t*>(col + i * kDispInPitch))));
      const int sexp = mx_scale_exp(m);
      const float r = mx_inv_scale(sexp);
      auto at = [&](int i) { return bf2f(*reinterpret_cast<const bf16_t*>(col + i * kDispInPitch)) * r; };
#pragma unroll
      for (int i = 0; i < 8; i++) q[i] = e4m3x4(at(4 * i), at(4 * i + 1), at(4 * i + 2), at(4 * i + 3));
      reinterpret_cast<uint8_t*>(s_csc)[lane * 4 + wave] = (uint8_t)(sexp + 127);
    }
    __syncthreads();  // every wave is done reading the bf16 tile
    {
      uint4* o = reinterpret_cast<uint4*>(s_buf + lane * kDispOutPitch + wave * 32);
      o[0] = make_uint4(q[0], q[1], q[2], q[3]);
      o[1] = make_uint4(q[4], q[5], q[6], q[7]);
    }
    __syncthreads();
    // the column scales of this tile: the four 32-row blocks of column c0 + lane are four
    // consecutive bytes, stored by wave 0 as one word (or as bytes when the rows per column
    // leave the word unaligned)
    if (wave == 0) {
      const int64_t sld = a.ld / kMxBlock;
      uint8_t* dst = a.s_cols + (int64_t)(c0 + lane) * sld + prow / kMxBlock;
      const uint32_t w = s_csc[lane];
      if (sld % 4 == 0) {
        *reinterpret_cast<uint32_t*>(dst) = w;
      } else {
#pragma unroll
        for (int b = 0; b < 4; b++) dst[b] = (uint8_t)(w >> (8 * b));
      }
    }
    // 64 columns x 128 bytes, 8 lanes per line
#pragma unroll
    for (int u = 0; u < kDispCols * kDispRows / 16 / kDispThreads; u++) {
      const int i = tid + kDispThreads * u, c = i >> 3, ch = i & 7;
      *reinterpret_cast<uint4*>(a.q_cols + (int64_t)(c0 + c) * a.ld + prow + ch * 16) =
          *reinterpret_cast<const uint4*>(s_buf + c * kDispOutPitch + ch * 16);
    }
    __syncthreads();  // the tile buffer is rewritten by the next column tile
#pragma unroll
    for (int i = 0; i < kDispChunks; i++) cur[i] = nxt[i];
  }
}

}  // namespace

hipError_t mx_dispatch(int R, int cols, int E, int k, const bf16_t* src, const int32_t* row_src,
                       const int32_t* offsets, const float* gates, const int32_t* slot_row, uint8_t* q_rows,
                       uint8_t* s_rows, uint8_t* q_cols, uint8_t* s_cols, hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (cols % kDispCols != 0 || E < 1 || E > kMaxExperts) return hipErrorInvalidValue;
  // upper bound of the padded row tiles: sum_e ceil(n_e / 128) <= ceil(R / 128) + E
  const int row_tiles = (R + kDispRows - 1) / kDispRows + E;
  const int col_tiles = cols / kDispCols;
  // about 2048 workgroups, each on a run of column tiles of one row tile
  int per = (int)(((int64_t)row_tiles * col_tiles + 2047) / 2048);
  per = per < 1 ? 1 : (per > col_tiles ? col_tiles : per);
  DispatchQ a{src, cols, row_src, offsets, E, gates, slot_row, k, q_rows, s_rows, q_cols, s_cols,
              (int64_t)R + (int64_t)kMxSegPad * E, per};
  const dim3 grid((unsigned)row_tiles, (unsigned)((col_tiles + per - 1) / per));
  hipLaunchKernelGGL(mx_dispatch_kernel, grid, dim3(kDispThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t mx_quantize_rows(int rows, int cols, const bf16_t* src, uint8_t* q, uint8_t* scales, hipStream_t st) {
  const int64_t n = (int64_t)rows * (cols / kMxBlock);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, rows, cols, src, q, scales,
                     0, 0);
  return hipGetLastError();
}

// W1 / W3 [E][f][cols] into one [E][2f][cols] code array whose 32-row blocks alternate
// W1, W3 (the column order of the forward GEMM's SwiGLU tiles)
static hipError_t mx_quantize_w13(int E, int f, int cols, const bf16_t* W1, const bf16_t* W3, uint8_t* q,
                                  uint8_t* scales, hipStream_t st) {
  const int64_t n = (int64_t)E * f * (cols / kMxBlock);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(mx_rows_kernel, grid, dim3(256), 0, st, E * f, cols, W1, q, scales, f, 0);
  hipLaunchKernelGGL(mx_rows_kernel, grid, dim3(256), 0, st, E * f, cols, W3, q, scales, f, 1);
  return hipGetLastError();
}

// total_tiles: upper bound of 128-row tiles (padded mode: rows_pad / 128; uniform mode:
// E * ceil(len / 128)); tiles past the device-side count exit at once.
static hipError_t launch_trans(TransQ a, int64_t total_tiles, hipStream_t st) {
  if (a.cols == 0 || total_tiles == 0) return hipSuccess;
  const unsigned gy = (unsigned)(total_tiles < 16384 ? total_tiles : 16384);
  dim3 grid((unsigned)((a.cols + kTransCols - 1) / kTransCols), gy);
  hipLaunchKernelGGL(mx_trans_kernel, grid, dim3(kTransThreads), 0, st, a);
  return hipGetLastError();
}

// Padded, per-segment transposed quantisation (rows grouped by seg_offsets).
hipError_t mx_quantize_cols_seg(int rows, int cols, const int32_t* seg_offsets, int nseg, const bf16_t* src,
                                uint8_t* q, uint8_t* scales, hipStream_t st) {
  const int rows_pad = rows + kMxSegPad * nseg;
  TransQ a{src, cols, cols, seg_offsets, nseg, 0, q, rows_pad, 0, scales, rows_pad / kMxBlock, 0, 0};
  return launch_trans(a, rows_pad / kTransRows, st);
}


// ---------------------------------------------------------------------------------------
// MXFP8 grouped GEMM: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and one E8M0
// scale per 32 elements along K.  Every operand arrives K-contiguous from the quantisers
// above (activations and forward weights row-wise, the forward weights of GEMM1 in the
// W1/W3 32-row interleave; weight-gradient operands transposed, per expert, 128-padded;
// backward weights transposed), so the kernel has one operand layout and every operand
// row range is linear.  Operand register layout of the instruction (per lane l,
// row/column l % 32, h = l / 32): bytes 0..15 hold k in [16h, 16h + 16), bytes 16..31
// hold k in [32 + 16h, 32 + 16h + 16); the lane's scale byte covers the 32-block h of
// the 64-deep step.
//
// Pipeline as in the bf16 kernel: the workgroup's tiles form one stream of 128-deep
// k-steps; each step's codes and scale words go straight from global memory into one of
// NS (2 or 3) LDS stage buffers, NS - 1 steps ahead of the MFMAs (bounded buffer loads:
// rows past an operand's end land as zeros); one barrier per step.
// ---------------------------------------------------------------------------------------
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void mx_lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// fp8 K-contiguous tile [BMN rows][TKB bytes] followed, in its stage buffer, by the
// step's scale words [BMN] (one dword per row: the E8M0 bytes of its four 32-blocks)
template <int BMN, int TKB, int NW>
struct MxOperand {
  static_assert(TKB == 128, "one scale dword per row and step");
  static constexpr int TILE_BYTES = BMN * TKB;
  static constexpr int SCALE_BYTES = BMN * 4;
  static constexpr int SEGS = TILE_BYTES / 1024;
  static constexpr int ROWS_PER_SEG = 1024 / TKB;
  static constexpr int CPR = TKB / 16;
  static constexpr int PER_THREAD = SEGS / NW;
  static constexpr int SCALE_SEGS = BMN / 64;  // 64 rows per scale load
  static_assert(SEGS % NW == 0, "every wave issues the same number of segments");

  static __device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

  // Scalar load state at the load cursor: per code segment of this wave its address and
  // readable bytes; the scale rows' address.  Set up per tile (begin), one add per step.
  struct Stream {
    const uint8_t* ptr[PER_THREAD];
    uint32_t bytes[PER_THREAD];
    uint32_t rb;                   // bytes per code row
    const uint8_t* sptr;           // scale word of row row0 at this step
    uint32_t srb;                  // bytes per scale row
    int rows;                      // valid rows from row0 (0: nothing is read)
  };
  template <class RowPtr, class ScalePtr>
  static __device__ __forceinline__ void begin(Stream& st, RowPtr rowptr, ScalePtr scaleptr, int row0, int row_end,
                                               int kt, int wave, bool live) {
    st.rb = (uint32_t)(rowptr(row0 + 1) - rowptr(row0));
    st.srb = (uint32_t)(scaleptr(row0 + 1) - scaleptr(row0));
    st.rows = live ? row_end - row0 : 0;
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) {
      const int r0 = row0 + (wave + NW * i) * ROWS_PER_SEG;
      st.ptr[i] = rowptr(r0) + kt;
      int valid = live ? row_end - r0 : 0;
      valid = valid < 0 ? 0 : (valid > ROWS_PER_SEG ? ROWS_PER_SEG : valid);
      st.bytes[i] = valid > 0 ? (uint32_t)(valid - 1) * st.rb + TKB : 0u;
    }
    st.sptr = scaleptr(row0) + kt / kMxBlock;
  }
  static __device__ __forceinline__ void next(Stream& st) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) st.ptr[i] += TKB;
    st.sptr += TKB / kMxBlock;
  }
  // codes and (waves sw0 .. sw0 + SCALE_SEGS - 1) scale words of the step into LDS
  static __device__ __forceinline__ void dma(const Stream& st, char* lds_tile, char* lds_scales, int wave, int lane,
                                             int sw0) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; i++) {
      const int s = wave + NW * i;
      const int r = lane / CPR, p = lane % CPR;
      const uint32_t voff = (uint32_t)r * st.rb + (uint32_t)(swz(s * ROWS_PER_SEG + r, p) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mx_rsrc(st.ptr[i], st.bytes[i]), (mx_lds_void_t*)(lds_tile + s * 1024),
                                               16, voff, 0, 0, 0);
    }
    const int j = wave - sw0;
    if (j >= 0 && j < SCALE_SEGS) {
      int valid = st.rows - 64 * j;
      valid = valid < 0 ? 0 : (valid > 64 ? 64 : valid);
      const uint32_t bytes = valid > 0 ? (uint32_t)(valid - 1) * st.srb + 4 : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mx_rsrc(st.sptr + (int64_t)64 * j * st.srb, bytes),
                                               (mx_lds_void_t*)(lds_scales + 256 * j), 4,
                                               (uint32_t)lane * st.srb, 0, 0, 0);
    }
  }
  // operand of 64-deep sub-step s for rows mn0 + lane % 32
  static __device__ __forceinline__ i32x8 frag(const char* lds, int s, int mn0, int lane) {
    const int r = mn0 + (lane & 31), h = lane >> 5;
    const v4i lo = *reinterpret_cast<const v4i*>(lds + r * TKB + (swz(r, 4 * s + h) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + r * TKB + (swz(r, 4 * s + 2 + h) << 4));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // the lane's scale byte of sub-step s (32-block 2 s + h of the step)
  static __device__ __forceinline__ int scale(const char* lds_scales, int s, int mn0, int lane) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(lds_scales + 4 * (mn0 + (lane & 31)));
    return (int)((w >> (8 * (2 * s + (lane >> 5)))) & 0xffu);
  }
};

}  // namespace

static inline size_t mx_dyn_lds_bytes(int E) { return (size_t)2 * (E + 1) * sizeof(int); }

template <class Cfg, class Prob, int TKB, int NS>
__global__ void __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(2)))
mx_gemm_kernel(const Prob p) {
  static_assert(NS == 2 || NS == 3, "two or three stage buffers");
  constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::NT;
  constexpr int WTM = Cfg::WTM, WTN = Cfg::WTN;
  constexpr int NW = NT / 64;
  using OA = MxOperand<BM, TKB, NW>;
  using OB = MxOperand<BN, TKB, NW>;
  constexpr int B_OFF = OA::TILE_BYTES, SA_OFF = B_OFF + OB::TILE_BYTES, SB_OFF = SA_OFF + OA::SCALE_BYTES;
  constexpr int STAGE_BYTES = SB_OFF + OB::SCALE_BYTES;
  static_assert(OA::SCALE_SEGS + OB::SCALE_SEGS <= NW, "one scale load per wave");
  // NS stage buffers as separate objects (the compiler then waits only for the loads a
  // buffer read depends on)
  __shared__ __attribute__((aligned(1024))) char sm0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sm1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sm2[NS == 3 ? STAGE_BYTES : 16];
  extern __shared__ __attribute__((aligned(16))) int s_dyn[];
  const int E = p.E;
  int* s_map = s_dyn;
  int* s_seg = s_dyn + E + 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave / Cfg::WAVES_N, wave_n = wave % Cfg::WAVES_N;
  // group starts: routed rows (Group::M) or 128-padded reduction starts (Group::K)
  if constexpr (Prob::GROUP == Group::M) {
    for (int e = tid; e <= E; e += NT) s_seg[e] = p.offsets[e];
  } else {
    for (int e = tid; e < E; e += NT)
      s_seg[e + 1] = (p.offsets[e + 1] - p.offsets[e] + kMxSegPad - 1) / kMxSegPad * kMxSegPad;
    __syncthreads();
    if (tid < kWave) {  // inclusive scan of the padded lengths by wave 0
      int carry = 0;
      for (int base = 1; base <= E; base += kWave) {
        const int e = base + lane;
        const int x = e <= E ? s_seg[e] : 0;
        int incl = x;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += y;
        }
        if (e <= E) s_seg[e] = carry + incl;
        carry += __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) s_seg[0] = 0;
    }
  }
  __syncthreads();
  auto seg = [&](int e) { return s_seg[e]; };
  const int total_tiles = build_tile_map<Prob::GROUP, BM, BN, NT>(s_map, seg, E, p.M, p.N, tid);
  const int G = gridDim.x;
  const int wg = xcd_logical_wg();
  if (wg >= total_tiles) return;  // uniform over the workgroup

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
  // load cursor (tile, k) and the operands' address streams at it
  struct Cursor {
    int t, k;
    TileRange tr;
  };
  Cursor lc;
  lc.t = wg;
  lc.tr = tile(wg);
  lc.k = lc.tr.k_beg;
  typename OA::Stream sa;
  typename OB::Stream sb;
  auto begin_streams = [&]() {
    const TileRange& r = lc.tr;
    const bool live = lc.t < total_tiles && lc.k < r.k_end;
    OA::begin(sa, [&](int x) { return p.a_row(r.e, x); }, [&](int x) { return p.a_scale_row(r.e, x); }, r.m0, r.m_end,
              lc.k, wave, live);
    OB::begin(sb, [&](int x) { return p.b_row(r.e, x); }, [&](int x) { return p.b_scale_row(r.e, x); }, r.n0, p.N,
              lc.k, wave, live);
  };
  auto advance = [&]() {
    lc.k += TKB;
    if (lc.k >= lc.tr.k_end) {
      lc.t += G;
      if (lc.t < total_tiles) lc.tr = tile(lc.t);
      lc.k = lc.tr.k_beg;
      begin_streams();
    } else {
      OA::next(sa);
      OB::next(sb);
    }
  };
  begin_streams();
  auto load_stage = [&](char* base) {
    OA::dma(sa, base, base + SA_OFF, wave, lane, 0);
    OB::dma(sb, base + B_OFF, base + SB_OFF, wave, lane, OA::SCALE_SEGS);
    advance();
  };
  // this wave's loads into buf have landed, then every wave meets
  auto ready = [&](const char* buf) {
    typedef __attribute__((address_space(3))) const volatile int lds_int_t;
    const int v = *(lds_int_t*)(buf + lane * 4);
    asm volatile("s_waitcnt lgkmcnt(0)" ::"v"(v) : "memory");
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
  // MFMAs of one 128-deep step (two 64-deep sub-steps), fragments double-buffered
  auto compute = [&](const char* st) {
    constexpr int KS = TKB / 64;
    i32x8 af[2][WTM], bfr[2][WTN];
    int xa[2][WTM], xb[2][WTN];
    auto read = [&](int s, int b) {
#pragma unroll
      for (int i = 0; i < WTM; i++) {
        af[b][i] = OA::frag(st, s, (wave_m * WTM + i) * 32, lane);
        xa[b][i] = OA::scale(st + SA_OFF, s, (wave_m * WTM + i) * 32, lane);
      }
#pragma unroll
      for (int j = 0; j < WTN; j++) {
        bfr[b][j] = OB::frag(st + B_OFF, s, (wave_n * WTN + j) * 32, lane);
        xb[b][j] = OB::scale(st + SB_OFF, s, (wave_n * WTN + j) * 32, lane);
      }
    };
    read(0, 0);
#pragma unroll
    for (int s = 0; s < KS; s++) {
      if (s + 1 < KS) read(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < WTM; i++)
#pragma unroll
        for (int j = 0; j < WTN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[s & 1][i], bfr[s & 1][j], acc[i][j], 0, 0, 0,
                                                                       xa[s & 1][i], 0, xb[s & 1][j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto steps_of = [&](const TileRange& r) {
    const int n = (r.k_end - r.k_beg + TKB - 1) / TKB;
    return n < 1 ? 1 : n;
  };

  int ct = wg;
  TileRange ctr = lc.tr;
  int ncs = steps_of(ctr), cs = 0;
  zero_acc();
  bool done = false;
  auto finish_step = [&]() {
    if (++cs == ncs) {
      tile_epilogue<Prob, WTM, WTN>(p, acc, ctr, wave_m, wave_n, lane);
      ct += G;
      if (ct < total_tiles) {
        ctr = tile(ct);
        ncs = steps_of(ctr);
        cs = 0;
        zero_acc();
      } else {
        done = true;
      }
    }
  };
  // step s is loaded into buffer s % NS, NS - 1 steps ahead (into the buffer the step
  // before read, once every wave is past this step's barrier); one exit, at the bottom
  load_stage(sm0);
  if constexpr (NS == 2) {
    for (;;) {
      ready(sm0);
      load_stage(sm1);
      compute(sm0);
      finish_step();
      ready(sm1);
      load_stage(sm0);
      compute(sm1);
      if (!done) finish_step();
      if (done) break;
    }
    return;
  }
  load_stage(sm1);
  for (;;) {
    ready(sm0);
    load_stage(sm2);
    compute(sm0);
    finish_step();
    ready(sm1);
    load_stage(sm0);
    compute(sm1);
    if (!done) finish_step();
    ready(sm2);
    load_stage(sm1);
    compute(sm2);
    if (!done) finish_step();
    if (done) break;
  }
}

// ---------------------------------------------------------------------------------------
// Problems.  Codes q* [rows][K] and scales s* [rows][K/32] (K-contiguous).
// ---------------------------------------------------------------------------------------
struct MxBase {
  static constexpr bool MXQ = false;  // no MXFP8 copy of the output
  static constexpr bool N_MAJOR = true;  // Group::M tile order within an expert
  static constexpr bool STORE16 = false;  // bf16 output rows through out_row (Epi::Store)
  int M = 0, N = 0, K = 0, E = 1;
  const int* offsets = nullptr;
  const uint8_t *qa = nullptr, *sa = nullptr;  // A codes / scales, row length K (padded for Group::K)
  int64_t lda = 0;                             // bytes per A row (= K)
};

struct MxGemm1 : MxBase {  // [a | b] = X [W1 | W3]^T, SwiGLU epilogue
  static constexpr Group GROUP = Group::M;
  static constexpr Epi EPI = Epi::SwiGLU;
  int f = 0;
  const uint8_t *qb = nullptr, *sb = nullptr;  // [E][2f][d]: 32-row blocks alternate W1, W3
  bf16_t *ab = nullptr, *h = nullptr;
  __device__ const uint8_t* a_row(int, int m) const { return qa + (int64_t)m * K; }
  __device__ const uint8_t* a_scale_row(int, int m) const { return sa + (int64_t)m * (K / kMxBlock); }
  __device__ const uint8_t* b_row(int e, int n) const { return qb + ((int64_t)e * N + n) * K; }
  __device__ const uint8_t* b_scale_row(int e, int n) const { return sb + ((int64_t)e * N + n) * (K / kMxBlock); }
  __device__ void epilogue_swiglu4(int m, int hcol, const float (&a)[4], const float (&b)[4]) const {
    bf16_t* abr = ab + (int64_t)m * 2 * f;
    store_bf16x4(abr + hcol, a);
    store_bf16x4(abr + f + hcol, b);
    float hv[4];
#pragma unroll
    for (int c = 0; c < 4; c++) hv[c] = a[c] * sigmoidf_(a[c]) * b[c];
    store_bf16x4(h + (int64_t)m * f + hcol, hv);
  }
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
  static constexpr bool STORE16 = true;
  __device__ bf16_t* out_row(int, int m) const { return C + (int64_t)m * N; }
  __device__ void epilogue4(int, int m, int n, const float (&v)[4]) const { store_bf16x4(C + (int64_t)m * N + n, v); }
};

struct MxDgrad2 : MxPlain {  // dh = dy W2_e, then the SwiGLU gradient from the saved a, b
  static constexpr Epi EPI = Epi::DSwiGLU;
  static constexpr bool N_MAJOR = false;  // as the bf16 dgrad2
  static constexpr bool STORE16 = false;  // 8-byte SwiGLU-gradient stores (epilogue4_pre)
  const bf16_t* ab = nullptr;
  bf16_t* dab = nullptr;
  __device__ AbPair prefetch4(int m, int n) const { return load_ab4(ab, N, m, n); }
  __device__ void epilogue4_pre(int, int m, int n, const float (&dh)[4], const AbPair& pr) const {
    dswiglu_store4(dab, N, m, n, dh, pr);
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
  static constexpr bool STORE16 = true;
  __device__ bf16_t* out_row(int e, int m) const {
    return m < split ? C0 + ((int64_t)e * split + m) * N : C1 + ((int64_t)e * (M - split) + (m - split)) * N;
  }
  __device__ void epilogue4(int e, int m, int n, const float (&v)[4]) const { store_bf16x4(out_row(e, m) + n, v); }
};

template <class Cfg, int NS, class Prob>
static hipError_t launch_mx_cfg(const Prob& p, hipStream_t st) {
  const auto kern = mx_gemm_kernel<Cfg, Prob, 128, NS>;
  const size_t dyn = mx_dyn_lds_bytes(p.E);
  // occupancy depends on the dynamic LDS, i.e. on E (cached per size)
  const int occ = kernel_occupancy(reinterpret_cast<const void*>(kern), Cfg::NT, dyn);
  int64_t bound;
  const int64_t ntn = (p.N + Cfg::BN - 1) / Cfg::BN;
  if constexpr (Prob::GROUP == Group::M) bound = ((int64_t)p.M / Cfg::BM + p.E) * ntn;
  else bound = (int64_t)p.E * ((p.M + Cfg::BM - 1) / Cfg::BM) * ntn;
  int64_t G = (int64_t)device_cu_count() * occ;
  if (bound < G) G = bound;
  G = ((G + 7) / 8) * 8;
  if (G < 8) G = 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(Cfg::NT), dyn, st, p);
  return hipGetLastError();
}

// Tiles: over long expert segments (1024 rows per expert or more on average: the M range of
// the forward and data-gradient GEMMs, the padded reduction of the weight-gradient ones)
// every MXFP8 GEMM takes 256 x 256 tiles in two stage buffers, otherwise 128 x 256 in
// three.  On MI355X at 2048 rows per expert the large tiles are 7-16% faster on each of the
// six.  MOE_MX_TILE=128x256 / 256x256 overrides the choice.
template <class Prob>
static hipError_t launch_mx(const Prob& p, hipStream_t st) {
  const int64_t rows = Prob::GROUP == Group::M ? p.M : p.K;
  bool big = rows >= (int64_t)1024 * p.E;
  if (const char* v = tuning_env("MOE_MX_TILE")) big = strcmp(v, "256x256") == 0;
  if (big) return launch_mx_cfg<TileCfg<256, 256, 2, 4>, 2>(p, st);
  return launch_mx_cfg<TileCfg<128, 256, 2, 4>, 3>(p, st);
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
                        bf16_t* ab, bf16_t* h, void* ws, hipStream_t st, MxIn x_rows) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ef = (int64_t)s.E * s.f;
  uint8_t *xq = c.take((size_t)s.R * s.d), *xs = c.take((size_t)s.R * s.d / kMxBlock);
  uint8_t *q13 = c.take((size_t)2 * Ef * s.d), *s13 = c.take((size_t)2 * Ef * s.d / kMxBlock);
  hipError_t err;
  if (x_rows.q) {
    xq = const_cast<uint8_t*>(x_rows.q);
    xs = const_cast<uint8_t*>(x_rows.s);
  } else if ((err = mx_quantize_rows(s.R, s.d, X, xq, xs, st)) != hipSuccess) {
    return err;
  }
  if ((err = mx_quantize_w13(s.E, s.f, s.d, W1, W3, q13, s13, st)) != hipSuccess) return err;
  MxGemm1 p;
  p.M = s.R; p.N = 2 * s.f; p.K = s.d; p.E = s.E; p.offsets = offsets; p.qa = xq; p.sa = xs; p.f = s.f;
  p.qb = q13; p.sb = s13; p.ab = ab; p.h = h;
  return launch_mx(p, st);
}

hipError_t gemm2_fwd_mx(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* W2, bf16_t* Y,
                        void* ws, hipStream_t st, MxIn h_rows) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ed = (int64_t)s.E * s.d;
  uint8_t *hq = c.take((size_t)s.R * s.f), *hs = c.take((size_t)s.R * s.f / kMxBlock);
  uint8_t *wq = c.take((size_t)Ed * s.f), *wsc = c.take((size_t)Ed * s.f / kMxBlock);
  hipError_t err;
  if (h_rows.q) {
    hq = const_cast<uint8_t*>(h_rows.q);
    hs = const_cast<uint8_t*>(h_rows.s);
  } else if ((err = mx_quantize_rows(s.R, s.f, H, hq, hs, st)) != hipSuccess) {
    return err;
  }
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
           (int64_t)cols * (k_len / kMxBlock), col_off};
  return launch_trans(a, (int64_t)E * ((rows_e + kTransRows - 1) / kTransRows), st);
}

hipError_t dgrad2_mx(const GemmShape& s, const int* offsets, const bf16_t* dY, const bf16_t* W2, const bf16_t* ab,
                     bf16_t* dab, void* ws, hipStream_t st, MxIn dy_rows) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ef = (int64_t)s.E * s.f;
  uint8_t *yq = c.take((size_t)s.R * s.d), *ys = c.take((size_t)s.R * s.d / kMxBlock);
  uint8_t *wq = c.take((size_t)Ef * s.d), *wsc = c.take((size_t)Ef * s.d / kMxBlock);
  hipError_t err;
  if (dy_rows.q) {
    yq = const_cast<uint8_t*>(dy_rows.q);
    ys = const_cast<uint8_t*>(dy_rows.s);
  } else if ((err = mx_quantize_rows(s.R, s.d, dY, yq, ys, st)) != hipSuccess) {
    return err;
  }
  if ((err = quantize_weight_t(s.E, s.d, s.f, W2, wq, wsc, s.d, 0, st)) != hipSuccess) return err;  // W2_e^T [f][d]
  MxDgrad2 p;
  p.M = s.R; p.N = s.f; p.K = s.d; p.E = s.E; p.offsets = offsets; p.qa = yq; p.sa = ys;
  p.qb = wq; p.sb = wsc; p.ab = ab; p.dab = dab;
  return launch_mx(p, st);
}

hipError_t dgrad1_mx(const GemmShape& s, const int* offsets, const bf16_t* dab, const bf16_t* W1, const bf16_t* W3,
                     bf16_t* dX, void* ws, hipStream_t st, MxIn dab_rows) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Ed = (int64_t)s.E * s.d;
  uint8_t *gq = c.take((size_t)s.R * 2 * s.f), *gs = c.take((size_t)s.R * 2 * s.f / kMxBlock);
  uint8_t *wq = c.take((size_t)Ed * 2 * s.f), *wsc = c.take((size_t)Ed * 2 * s.f / kMxBlock);
  hipError_t err;
  if (dab_rows.q) {
    gq = const_cast<uint8_t*>(dab_rows.q);
    gs = const_cast<uint8_t*>(dab_rows.s);
  } else if ((err = mx_quantize_rows(s.R, 2 * s.f, dab, gq, gs, st)) != hipSuccess) {
    return err;
  }
  // [W1_e ; W3_e]^T = [d][2f]: W1_e^T in columns [0, f), W3_e^T in [f, 2f)
  if ((err = quantize_weight_t(s.E, s.f, s.d, W1, wq, wsc, 2 * s.f, 0, st)) != hipSuccess) return err;
  if ((err = quantize_weight_t(s.E, s.f, s.d, W3, wq, wsc, 2 * s.f, s.f, st)) != hipSuccess) return err;
  MxPlain p;
  p.M = s.R; p.N = s.d; p.K = 2 * s.f; p.E = s.E; p.offsets = offsets; p.qa = gq; p.sa = gs;
  p.qb = wq; p.sb = wsc; p.C = dX;
  return launch_mx(p, st);
}

hipError_t wgrad2_mx(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* dY, bf16_t* dW2,
                     void* ws, hipStream_t st, MxIn dy_cols) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Rp = (int64_t)s.R + (int64_t)kMxSegPad * s.E;
  uint8_t *aq = c.take((size_t)(s.d * Rp)), *as = c.take((size_t)(s.d * Rp / kMxBlock));
  uint8_t *bq = c.take((size_t)(s.f * Rp)), *bs = c.take((size_t)(s.f * Rp / kMxBlock));
  hipError_t err;
  if (dy_cols.q) {
    aq = const_cast<uint8_t*>(dy_cols.q);
    as = const_cast<uint8_t*>(dy_cols.s);
  } else if ((err = mx_quantize_cols_seg(s.R, s.d, offsets, s.E, dY, aq, as, st)) != hipSuccess) {
    return err;
  }
  if ((err = mx_quantize_cols_seg(s.R, s.f, offsets, s.E, H, bq, bs, st)) != hipSuccess) return err;
  MxWgrad p;
  p.M = s.d; p.N = s.f; p.K = (int)Rp; p.E = s.E; p.offsets = offsets; p.qa = aq; p.sa = as;
  p.qb = bq; p.sb = bs; p.C0 = dW2; p.split = s.d;
  return launch_mx(p, st);
}

hipError_t wgrad1_mx(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* dab, bf16_t* dW1,
                     bf16_t* dW3, void* ws, hipStream_t st, MxIn x_cols) {
  Carve c{static_cast<char*>(ws)};
  const int64_t Rp = (int64_t)s.R + (int64_t)kMxSegPad * s.E;
  uint8_t *aq = c.take((size_t)(2 * s.f * Rp)), *as = c.take((size_t)(2 * s.f * Rp / kMxBlock));
  uint8_t *bq = c.take((size_t)(s.d * Rp)), *bs = c.take((size_t)(s.d * Rp / kMxBlock));
  hipError_t err;
  if ((err = mx_quantize_cols_seg(s.R, 2 * s.f, offsets, s.E, dab, aq, as, st)) != hipSuccess) return err;
  if (x_cols.q) {
    bq = const_cast<uint8_t*>(x_cols.q);
    bs = const_cast<uint8_t*>(x_cols.s);
  } else if ((err = mx_quantize_cols_seg(s.R, s.d, offsets, s.E, X, bq, bs, st)) != hipSuccess) {
    return err;
  }
  MxWgrad p;
  p.M = 2 * s.f; p.N = s.d; p.K = (int)Rp; p.E = s.E; p.offsets = offsets; p.qa = aq; p.sa = as;
  p.qb = bq; p.sb = bs; p.C0 = dW1; p.C1 = dW3; p.split = s.f;
  return launch_mx(p, st);
}

}  // namespace moe
