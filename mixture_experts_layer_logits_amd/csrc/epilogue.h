// Tile epilogue shared by the grouped GEMM kernels (bf16 and MXFP8 operands).
//
// A 32x32 MFMA accumulator block leaves lane l with column l % 32 and, in register r,
// row 8 (r / 4) + 4 (l / 32) + r % 4: every lane holds 16 rows of one column.  A 4x4
// transpose inside each lane quad (two DPP exchanges) turns each group of 4 registers
// into one row and 4 consecutive columns per lane, so the outputs leave as 8-byte bf16
// stores (8 rows x 64 contiguous bytes per store instruction) instead of 2-byte ones.
//
// Problems with bf16 outputs (STORE16) go one step further: the two lanes of each quad pair
// (quads 2c and 2c + 1) swap four columns, so each lane holds 8 consecutive columns of one
// row and stores 16 bytes (16 rows x 64 bytes per instruction).  On MI355X 16-byte stores
// of this shape write ~1.5x faster than 8-byte ones (6.3-6.8 against 4.0-4.3 TB/s over
// 256 CUs); the bytes written are the same.
//
// Problem interface (all columns n are multiples of 4; rows m < m_end, n < N are checked
// here, partial column groups are the problem's business):
//   Epi::Store                 p.epilogue4(e, m, n, v[4])          columns n .. n+3
//   Epi::Store, STORE16        p.out_row(e, m) -> bf16 row; 16-byte stores at columns
//                              n .. n+7 (N a multiple of 8)
//   Epi::SwiGLU, STORE16       p.swiglu4(a[4], b[4], h[4]), then p.store_swiglu16(m, hcol,
//                              a, b, h) with 8 packed bf16 columns each (and, MXQ,
//                              p.store_swiglu16_q(m, hcol, h, valid, first) from every lane)
//   Epi::DSwiGLU, STORE16      p.prefetch4 as above, then p.store_dswiglu16(m, n, da, db)
//                              (and, MXQ, p.store_dswiglu16_q(m, n, da, db, valid, first))
//   Epi::SwiGLU                p.epilogue_swiglu4(m, hcol, a[4], b[4])
//   Epi::DSwiGLU               p.prefetch4(m, n) -> AbPair, then p.epilogue4_pre(e, m, n, v[4], pair)
// A problem with MXQ = true also writes its SwiGLU (h) or SwiGLU-gradient (da | db) output as
// MXFP8 row blocks; its _q epilogue is called by every lane (the block maximum is a shuffle
// over the 8 lanes of the block) with `valid` gating the stores:
//   Epi::SwiGLU                p.epilogue_swiglu4_q(m, hcol, a[4], b[4], valid, quad)
//   Epi::DSwiGLU               p.epilogue4_pre_q(e, m, n, v[4], pair, valid, quad)
// The SwiGLU gradient reads the saved a, b of every output position.  Those loads are issued
// for a whole 32-row block of the wave before any of its stores: memory operations complete
// in order on one counter, so a load issued after a store (or after the operand loads still
// in flight for the next steps) would wait for all of them.
#pragma once
#include "common.h"
#include "gemm.h"
#include "mxcode.h"
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

// Saved a and b of four consecutive hidden columns of one row, packed bf16.
struct AbPair {
  uint2 a, b;
};
// ab [rows][2N] (a in columns [0, N), b in [N, 2N)): row m, columns n .. n+3
__device__ __forceinline__ AbPair load_ab4(const bf16_t* ab, int N, int m, int n) {
  const bf16_t* abr = ab + (int64_t)m * 2 * N;
  return AbPair{*reinterpret_cast<const uint2*>(abr + n), *reinterpret_cast<const uint2*>(abr + N + n)};
}
// da = dh b s (1 + a (1 - s)), db = dh silu(a), s = sigmoid(a)
__device__ __forceinline__ void dswiglu4(const float (&dh)[4], const AbPair& pr, float (&da)[4], float (&db)[4]) {
  float a[4], b[4];
  load_bf16x4(reinterpret_cast<const bf16_t*>(&pr.a), a);
  load_bf16x4(reinterpret_cast<const bf16_t*>(&pr.b), b);
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const float s = sigmoidf_(a[c]);
    da[c] = dh[c] * b[c] * s * (1.f + a[c] * (1.f - s));
    db[c] = dh[c] * a[c] * s;
  }
}
// ... stored bf16 to dab [rows][2N]
__device__ __forceinline__ void dswiglu_store4(bf16_t* dab, int N, int m, int n, const float (&dh)[4],
                                               const AbPair& pr) {
  float da[4], db[4];
  dswiglu4(dh, pr, da, db);
  bf16_t* o = dab + (int64_t)m * 2 * N;
  store_bf16x4(o + n, da);
  store_bf16x4(o + N + n, db);
}

// One MXFP8 row block of 32 consecutive outputs, held 4 per lane by the 8 lanes that share
// (lane & 3, lane >> 5) (quad = (lane & 31) >> 2 = 0..7): the values are rounded to bf16 as
// the bf16 copy stores them, their block maximum is taken over the 8 lanes (butterfly over
// lane bits 2-4), and each lane encodes its 4 values under the block's scale.  Bit for bit
// what the row quantiser writes for the stored bf16 row.  Every lane must call it; `valid`
// (uniform over the block's lanes) gates the stores of the 4 codes at q and, from quad 0,
// the scale byte at sc.
__device__ __forceinline__ void mx_block_store4(const float (&v)[4], bool valid, uint8_t* q, uint8_t* sc, int quad) {
  float r[4], amax = 0.f;
#pragma unroll
  for (int c = 0; c < 4; c++) {
    r[c] = bf2f(f2bf(v[c]));
    amax = fmaxf(amax, fabsf(r[c]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 8, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  const int s = mx_scale_exp(amax);
  const float inv = mx_inv_scale(s);
  const uint32_t codes = e4m3x4(r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv);
  if (valid) {
    *reinterpret_cast<uint32_t*>(q) = codes;
    if (quad == 0) *sc = (uint8_t)(s + 127);
  }
}

// Lanes of quads 2c and 2c + 1 after the quad transpose: w[h] is the packed bf16 of row group
// 2 pq + h at the lane's 4 columns.  Returns the 8 consecutive columns of the lane's own row
// group (2 pq for the even quad, 2 pq + 1 for the odd one): each lane sends its partner (lane
// ^ 4) the partner's row group.
__device__ __forceinline__ uint4 pair_row16(const uint32_t (&w)[2][2], bool odd) {
  const uint32_t r0 = __shfl_xor(odd ? w[0][0] : w[1][0], 4, kWave);
  const uint32_t r1 = __shfl_xor(odd ? w[0][1] : w[1][1], 4, kWave);
  return odd ? make_uint4(r0, r1, w[1][0], w[1][1]) : make_uint4(w[0][0], w[0][1], r0, r1);
}

// The MXFP8 row block of 32 columns held 8 per lane (packed bf16, the stored values) by the
// 4 lanes that differ only in lane bits 3 and 4: block maximum over those lanes, then each
// lane encodes its 8 values.  Bit for bit what the row quantiser writes for the stored row.
// Every lane must call it; `valid` gates the 8-byte code store at q and, from the block's
// first lane, the scale byte at sc.
__device__ __forceinline__ void mx_block_store8(const uint4& pk, bool valid, uint8_t* q, uint8_t* sc, bool first) {
  const uint32_t w[4] = {pk.x, pk.y, pk.z, pk.w};
  float r[8], amax = 0.f;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    r[2 * u] = __uint_as_float(w[u] << 16);
    r[2 * u + 1] = __uint_as_float(w[u] & 0xffff0000u);
  }
#pragma unroll
  for (int c = 0; c < 8; c++) amax = fmaxf(amax, fabsf(r[c]));
  amax = fmaxf(amax, __shfl_xor(amax, 8, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  const int s = mx_scale_exp(amax);
  const float inv = mx_inv_scale(s);
  const uint2 codes = make_uint2(e4m3x4(r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv),
                                 e4m3x4(r[4] * inv, r[5] * inv, r[6] * inv, r[7] * inv));
  if (valid) {
    *reinterpret_cast<uint2*>(q) = codes;
    if (first) *sc = (uint8_t)(s + 127);
  }
}

// Writes the tile of wave (wave_m, wave_n) whose accumulators are acc.
template <class Prob, int WTM, int WTN>
__device__ __forceinline__ void tile_epilogue(const Prob& p, const f32x16 (&acc)[WTM][WTN], const TileRange& tr,
                                              int wave_m, int wave_n, int lane) {
  const int sub = lane & 3, quad = (lane & 31) >> 2, half = lane >> 5;
#pragma unroll
  for (int i = 0; i < WTM; i++) {
    if constexpr (Prob::EPI == Epi::DSwiGLU) {
      // every saved (a, b) of the block first (rows and columns clamped into the tile, so no
      // load is out of range or under a branch), then the gradients and their stores
      AbPair pre[4][WTN];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        int m = tr.m0 + (wave_m * WTM + i) * 32 + 8 * q + 4 * half + sub;
        m = m < tr.m_end ? m : tr.m_end - 1;
#pragma unroll
        for (int j = 0; j < WTN; j++) {
          int n = tr.n0 + (wave_n * WTN + j) * 32 + 4 * quad;
          n = n < p.N ? n : p.N - 4;
          pre[q][j] = p.prefetch4(m, n);
        }
      }
      if constexpr (Prob::STORE16) {
        // the gradients of the lane's own 4 columns in fp32, rounded, then completed to 8
        // columns of one row by the quad-pair exchange: 16-byte stores
        const bool odd = quad & 1;
#pragma unroll
        for (int pq = 0; pq < 2; pq++) {
          const int m = tr.m0 + (wave_m * WTM + i) * 32 + 8 * (2 * pq + (odd ? 1 : 0)) + 4 * half + sub;
#pragma unroll
          for (int j = 0; j < WTN; j++) {
            uint32_t wa[2][2], wb[2][2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
              float v[4], da[4], db[4];
#pragma unroll
              for (int c = 0; c < 4; c++) v[c] = acc[i][j][4 * (2 * pq + h) + c];
              quad_transpose(v, lane);
              dswiglu4(v, pre[2 * pq + h][j], da, db);
              wa[h][0] = pack_bf16x2(da[0], da[1]);
              wa[h][1] = pack_bf16x2(da[2], da[3]);
              wb[h][0] = pack_bf16x2(db[0], db[1]);
              wb[h][1] = pack_bf16x2(db[2], db[3]);
            }
            const uint4 ua = pair_row16(wa, odd), ub = pair_row16(wb, odd);
            const int n = tr.n0 + (wave_n * WTN + j) * 32 + 8 * (quad >> 1);
            const bool valid = m < tr.m_end && n < p.N;
            if (valid) p.store_dswiglu16(m, n, ua, ub);
            if constexpr (Prob::MXQ) p.store_dswiglu16_q(m, n, ua, ub, valid, (quad >> 1) == 0);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int m = tr.m0 + (wave_m * WTM + i) * 32 + 8 * q + 4 * half + sub;
#pragma unroll
          for (int j = 0; j < WTN; j++) {
            float v[4];
#pragma unroll
            for (int c = 0; c < 4; c++) v[c] = acc[i][j][4 * q + c];
            quad_transpose(v, lane);
            const int n = tr.n0 + (wave_n * WTN + j) * 32 + 4 * quad;
            const bool valid = m < tr.m_end && n < p.N;
            if constexpr (Prob::MXQ) p.epilogue4_pre_q(tr.e, m, n, v, pre[q][j], valid, quad);
            else if (valid) p.epilogue4_pre(tr.e, m, n, v, pre[q][j]);
          }
        }
      }
    } else if constexpr (Prob::EPI == Epi::SwiGLU && Prob::STORE16) {
      // a and b of the lane's own 4 columns, h from them in fp32, all three rounded and
      // completed to 8 columns of one row by the quad-pair exchange: 16-byte stores
      const bool odd = quad & 1;
#pragma unroll
      for (int pq = 0; pq < 2; pq++) {
        const int m = tr.m0 + (wave_m * WTM + i) * 32 + 8 * (2 * pq + (odd ? 1 : 0)) + 4 * half + sub;
#pragma unroll
        for (int j = 0; j < WTN; j += 2) {
          uint32_t wa[2][2], wb[2][2], wh[2][2];
#pragma unroll
          for (int h = 0; h < 2; h++) {
            float a[4], b[4], hv[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
              a[c] = acc[i][j][4 * (2 * pq + h) + c];
              b[c] = acc[i][j + 1][4 * (2 * pq + h) + c];
            }
            quad_transpose(a, lane);
            quad_transpose(b, lane);
            p.swiglu4(a, b, hv);
            wa[h][0] = pack_bf16x2(a[0], a[1]);
            wa[h][1] = pack_bf16x2(a[2], a[3]);
            wb[h][0] = pack_bf16x2(b[0], b[1]);
            wb[h][1] = pack_bf16x2(b[2], b[3]);
            wh[h][0] = pack_bf16x2(hv[0], hv[1]);
            wh[h][1] = pack_bf16x2(hv[2], hv[3]);
          }
          const uint4 ua = pair_row16(wa, odd), ub = pair_row16(wb, odd), uh = pair_row16(wh, odd);
          const int hcol = tr.n0 / 2 + ((wave_n * WTN + j) >> 1) * 32 + 8 * (quad >> 1);
          const bool valid = m < tr.m_end && hcol < p.N / 2;
          if (valid) p.store_swiglu16(m, hcol, ua, ub, uh);
          if constexpr (Prob::MXQ) p.store_swiglu16_q(m, hcol, uh, valid, (quad >> 1) == 0);
        }
      }
    } else if constexpr (Prob::EPI == Epi::Store && Prob::STORE16) {
      // the even lane of a quad pair takes row group 2 pq, the odd lane 2 pq + 1; each sends
      // its partner the four columns of the partner's row group
      const bool odd = quad & 1;
#pragma unroll
      for (int pq = 0; pq < 2; pq++) {
        const int m = tr.m0 + (wave_m * WTM + i) * 32 + 8 * (2 * pq + (odd ? 1 : 0)) + 4 * half + sub;
#pragma unroll
        for (int j = 0; j < WTN; j++) {
          uint32_t w[2][2];  // packed bf16 of row groups 2 pq (w[0]) and 2 pq + 1 (w[1])
#pragma unroll
          for (int h = 0; h < 2; h++) {
            float v[4];
#pragma unroll
            for (int c = 0; c < 4; c++) v[c] = acc[i][j][4 * (2 * pq + h) + c];
            quad_transpose(v, lane);
            w[h][0] = pack_bf16x2(v[0], v[1]);
            w[h][1] = pack_bf16x2(v[2], v[3]);
          }
          const uint4 o = pair_row16(w, odd);
          const int n = tr.n0 + (wave_n * WTN + j) * 32 + 8 * (quad >> 1);
          if (m < tr.m_end && n < p.N) *reinterpret_cast<uint4*>(p.out_row(tr.e, m) + n) = o;
        }
      }
    } else {
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
            const bool valid = m < tr.m_end && hcol < p.N / 2;
            if constexpr (Prob::MXQ) p.epilogue_swiglu4_q(m, hcol, a, b, valid, quad);
            else if (valid) p.epilogue_swiglu4(m, hcol, a, b);
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
}

}  // namespace moe
