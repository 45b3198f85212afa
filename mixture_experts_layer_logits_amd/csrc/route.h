// Internal declarations: routing, dispatch and row-movement launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include "common.h"

namespace moe {

constexpr int kRouteChunk = 32;   // tokens per routing workgroup (stable-rank chunk)
constexpr int kMaxTopK = 32;      // largest supported k
constexpr int MOE_DEVERR_EXPERT_RANGE_BIT = 1;
constexpr int MOE_DEVERR_DUPLICATE_BIT = 2;

size_t route_workspace_bytes(int T, int E, int k);
// The allocation-free routing entry point's fixed device scratch: 2^20 int32 (4 MiB) per
// device; shapes whose route_workspace_bytes exceed it are refused.
constexpr size_t kRouteScratchInts = size_t(1) << 20;
// Device address of that scratch on the current device (taken once per device).
hipError_t route_scratch_ptr(int32_t** out);
hipError_t route_topk(int T, int E, int k, const float* logits, int32_t* idx, float* gates, int32_t* counts,
                      int32_t* offsets, int32_t* slot_row, void* ws, hipStream_t st);
hipError_t route_given(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                       int32_t* slot_row, int32_t* dev_err, void* ws, hipStream_t st);
hipError_t route_backward(int T, int E, int k, const float* dgates, const float* gates, const int32_t* idx,
                          float* dlogits, hipStream_t st);

// elem_bytes: 2 (bf16) or 4 (float)
hipError_t permute_rows(int elem_bytes, int T, int d, int k, const void* x, const int32_t* slot_row,
                        int32_t* row_src, void* x_perm, hipStream_t st);
hipError_t combine_rows(int elem_bytes, int T, int d, int k, const void* y_perm, const float* gates,
                        const int32_t* slot_row, const void* y_add, void* y, hipStream_t st);
hipError_t combine_rows_bwd(int elem_bytes, int T, int d, int k, const void* dy, const void* y_perm,
                            const float* gates, const int32_t* slot_row, void* dy_perm, float* dgates,
                            hipStream_t st);
// dgates[t, j] = <dy[t], y_perm[slot_row[t, j]]> (bf16 rows), bit-identical with combine_rows_bwd's
hipError_t dgates_rows(int T, int d, int k, const bf16_t* dy, const bf16_t* y_perm, const int32_t* slot_row,
                       float* dgates, hipStream_t st);
// row_src[slot_row[t, j]] = t
hipError_t row_src_rows(int T, int k, const int32_t* slot_row, int32_t* row_src, hipStream_t st);
hipError_t unpermute_sum_rows(int elem_bytes, int T, int d, int k, const void* dx_perm, const int32_t* slot_row,
                              const void* dx_r, const void* dx_add, void* dx, hipStream_t st);
// un-permute with the router's input gradient folded in (k rows of Wr per token)
hipError_t unpermute_router_rows(int elem_bytes, int T, int d, int k, int E, const void* dx_perm,
                                 const int32_t* slot_row, const int32_t* topk_idx, const float* dlogits,
                                 const void* Wr, const void* dx_add, void* dx, hipStream_t st);

}  // namespace moe
