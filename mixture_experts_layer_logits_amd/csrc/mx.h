// Internal declarations: MXFP8 (E4M3 elements, E8M0 scale per 32) quantisers and the
// scaled-MFMA expert GEMMs.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include "gemm.h"

namespace moe {

constexpr int kMxBlock = 32;     // elements per shared scale
constexpr int kMxSegPad = 128;   // expert segments are padded to this many rows in K-major copies

size_t mx_workspace_bytes(int R, int d, int f, int E);

// axis 0: blocks along rows; q [rows, cols], scales [rows, cols/32]
hipError_t mx_quantize_rows(int rows, int cols, const bf16_t* src, uint8_t* q, uint8_t* scales, hipStream_t st);
// axis 1: blocks down columns restarting at segment starts; transposed padded output
hipError_t mx_quantize_cols_seg(int rows, int cols, const int32_t* seg_offsets, int nseg, const bf16_t* src,
                                uint8_t* q, uint8_t* scales, hipStream_t st);

// MXFP8 dispatch: rows v_r = src[row_src[r]] (gates == nullptr) or bf16(gates[t, j] * src[t])
// for r = slot_row[t, j], written only as codes in the row layout [R][cols] (+ scales
// [R][cols/32]) and the per-expert padded column layout [cols][R + 128 E] (+ scales)
hipError_t mx_dispatch(int R, int cols, int E, int k, const bf16_t* src, const int32_t* row_src,
                       const int32_t* offsets, const float* gates, const int32_t* slot_row, uint8_t* q_rows,
                       uint8_t* s_rows, uint8_t* q_cols, uint8_t* s_cols, hipStream_t st);

// An activation operand the caller has already quantised (by the MXFP8 dispatch, or by the
// epilogue of the bf16 GEMM that produced it), in the layout the GEMM reads; q == nullptr:
// the GEMM quantises its bf16 source itself.
struct MxIn {
  const uint8_t* q = nullptr;
  const uint8_t* s = nullptr;
};

hipError_t gemm1_fwd_mx(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* W1, const bf16_t* W3,
                        bf16_t* ab, bf16_t* h, void* ws, hipStream_t st, MxIn x_rows = {});
hipError_t gemm2_fwd_mx(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* W2, bf16_t* Y,
                        void* ws, hipStream_t st, MxIn h_rows = {});
hipError_t dgrad2_mx(const GemmShape& s, const int* offsets, const bf16_t* dY, const bf16_t* W2, const bf16_t* ab,
                     bf16_t* dab, void* ws, hipStream_t st, MxIn dy_rows = {});
hipError_t wgrad2_mx(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* dY, bf16_t* dW2,
                     void* ws, hipStream_t st, MxIn dy_cols = {});
hipError_t dgrad1_mx(const GemmShape& s, const int* offsets, const bf16_t* dab, const bf16_t* W1, const bf16_t* W3,
                     bf16_t* dX, void* ws, hipStream_t st, MxIn dab_rows = {});
hipError_t wgrad1_mx(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* dab, bf16_t* dW1,
                     bf16_t* dW3, void* ws, hipStream_t st, MxIn x_cols = {});

}  // namespace moe
