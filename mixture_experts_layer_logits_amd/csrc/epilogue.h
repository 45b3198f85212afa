// Tile epilogue shared by the grouped GEMM kernels (bf16 and MXFP8 operands).
//
// A 32x32 MFMA accumulator block leaves lane l with column l % 32 and, in register r,
// row 8 (r / 4) + 4 (l / 32) + r % 4: every lane holds 16 rows of one column.  A 4x4
// transpose inside each lane quad (two DPP exchanges) turns each group of 4 registers
// into one row and 4 consecutive columns per lane, so the outputs leave as 8-byte bf16
// stores (8 rows x 64 contiguous bytes per store instruction) instead of 2-byte ones.
//
// Problem interface (all columns n are multiples of 4; rows m < m_end, n < N are checked
// here, partial column groups are the problem's business):
//   Epi::Store, Epi::DSwiGLU   p.epilogue4(e, m, n, v[4])          columns n .. n+3
//   Epi::SwiGLU                p.epilogue_swiglu4(m, hcol, a[4], b[4])
#pragma once
#include "common.h"
#include "gemm.h"
#include "tilemap.h"

namespace moe {

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// On entry lane s (= lane % 4) of each quad holds x[r] = C(row r, column s) of a 4x4
// block; on exit x[c] = C(row s, column c).
__device__ __forceinline__ void quad_transpose(float (&x)[4], int lane) {
  constexpr int kSwap2 = 0x4E;  // quad_perm [2,3,0,1]: exchange with lane ^ 2
  constexpr int kSwap1 = 0xB1;  // quad_perm [1,0,3,2]: exchange with lane ^ 1
  const bool hi = lane & 2, odd = lane & 1;
  // exchange 2x2 sub-blocks with lane ^ 2: lane s then holds rows 2(s/2), 2(s/2)+1 at
  // columns s % 2 (z0, z1) and s % 2 + 2 (z2, z3)
  const float r0 = dpp_f<kSwap2>(hi ? x[0] : x[2]);
  const float r1 = dpp_f<kSwap2>(hi ? x[1] : x[3]);
  const float z0 = hi ? r0 : x[0], z1 = hi ? r1 : x[1];
  const float z2 = hi ? x[2] : r0, z3 = hi ? x[3] : r1;
  // exchange single elements with lane ^ 1: lane s keeps row s
  const float q0 = dpp_f<kSwap1>(odd ? z0 : z1);
  const float q1 = dpp_f<kSwap1>(odd ? z2 : z3);
  x[0] = odd ? q0 : z0;
  x[1] = odd ? z1 : q0;
  x[2] = odd ? q1 : z2;
  x[3] = odd ? z3 : q1;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void store_bf16x4(bf16_t* p, const float (&v)[4]) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void load_bf16x4(const bf16_t* p, float (&v)[4]) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}

// Writes the tile of wave (wave_m, wave_n) whose accumulators are acc.
template <class Prob, int WTM, int WTN>
__device__ __forceinline__ void tile_epilogue(const Prob& p, const f32x16 (&acc)[WTM][WTN], const TileRange& tr,
                                              int wave_m, int wave_n, int lane) {
  const int sub = lane & 3, quad = (lane & 31) >> 2, half = lane >> 5;
#pragma unroll
  for (int i = 0; i < WTM; i++) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int m = tr.m0 + (wave_m * WTM + i) * 32 + 8 * q + 4 * half + sub;
      if constexpr (Prob::EPI == Epi::SwiGLU) {
        // 32-column blocks alternate a (even j) and b (odd j) of the same h columns
#pragma unroll
        for (int j = 0; j < WTN; j += 2) {
          float a[4], b[4];
#pragma unroll
          for (int c = 0; c < 4; c++) {
            a[c] = acc[i][j][4 * q + c];
            b[c] = acc[i][j + 1][4 * q + c];
          }
          quad_transpose(a, lane);
          quad_transpose(b, lane);
          const int hcol = tr.n0 / 2 + ((wave_n * WTN + j) >> 1) * 32 + 4 * quad;
          if (m < tr.m_end && hcol < p.N / 2) p.epilogue_swiglu4(m, hcol, a, b);
        }
      } else {
#pragma unroll
        for (int j = 0; j < WTN; j++) {
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; c++) v[c] = acc[i][j][4 * q + c];
          quad_transpose(v, lane);
          const int n = tr.n0 + (wave_n * WTN + j) * 32 + 4 * quad;
          if (m < tr.m_end && n < p.N) p.epilogue4(tr.e, m, n, v);
        }
      }
    }
  }
}

}  // namespace moe
