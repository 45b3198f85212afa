// Internal declarations of the grouped-GEMM launchers (bf16 MFMA, fp32 reference-grade
// FMA, MXFP8 scaled MFMA).  Not part of the public C-ABI.
#pragma once
#include <hip/hip_runtime.h>
#include "common.h"

namespace moe {

constexpr int kMaxExperts = 1024;

enum class Group { M, K };
enum class Epi { Store, SwiGLU, DSwiGLU };

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M / 32, WTN = BN / WAVES_N / 32;
};

// Host-side launch state (capi.cpp).  Every cache is filled once and safe to read and fill
// from several host threads at once.
// Compute units of the current device (cached per device).
int device_cu_count();
// Resident workgroups per compute unit of `kern` at `threads` threads and `dyn_lds` bytes of
// dynamic LDS on the current device (at least 1; cached per device, kernel and sizes).
int kernel_occupancy(const void* kern, int threads, size_t dyn_lds);
// A tuning override from the environment (MOE_TILE_*, MOE_GEMM_*, MOE_MX_TILE), read at the
// first request of each name and kept for the life of the process; nullptr when unset.
const char* tuning_env(const char* name);

// Expert-GEMM sizes: R routed rows, d model width, f hidden width, E experts.
struct GemmShape {
  int R, d, f, E;
};

// bf16 grouped GEMMs (offsets: device [E+1] segment starts)
// hq, hs (optional): h also written as MXFP8 row blocks (codes [R][f], scales [R][f/32])
hipError_t gemm1_fwd_bf16(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* W1,
                          const bf16_t* W3, bf16_t* ab, bf16_t* h, hipStream_t st, uint8_t* hq = nullptr,
                          uint8_t* hs = nullptr);
hipError_t gemm2_fwd_bf16(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* W2, bf16_t* Y,
                          hipStream_t st);
// dq, ds (optional): [da | db] also written as MXFP8 row blocks (codes [R][2f], scales [R][2f/32])
hipError_t dgrad2_bf16(const GemmShape& s, const int* offsets, const bf16_t* dY, const bf16_t* W2,
                       const bf16_t* ab, bf16_t* dab, hipStream_t st, uint8_t* dq = nullptr,
                       uint8_t* ds = nullptr);
// weight gradients; with a single group (E == 1) and ws of wgrad_split_workspace_bytes
// the reduction over the rows is split (ws may be null: no split)
hipError_t wgrad2_bf16(const GemmShape& s, const int* offsets, const bf16_t* H, const bf16_t* dY, bf16_t* dW2,
                       void* ws, hipStream_t st);
hipError_t dgrad1_bf16(const GemmShape& s, const int* offsets, const bf16_t* dab, const bf16_t* W1,
                       const bf16_t* W3, bf16_t* dX, hipStream_t st);
hipError_t wgrad1_bf16(const GemmShape& s, const int* offsets, const bf16_t* X, const bf16_t* dab, bf16_t* dW1,
                       bf16_t* dW3, void* ws, hipStream_t st);
size_t wgrad_split_workspace_bytes(const GemmShape& s);
// router GEMMs (single group)
hipError_t router_fwd_bf16(int T, int d, int E, const bf16_t* X, const bf16_t* Wr, const float* bias, float* L,
                           hipStream_t st);
// dx_r = dlogits Wr, dWr = dlogits^T x (workspace: router_dw_workspace_bytes)
hipError_t router_bwd_bf16(int T, int d, int E, const float* dL, const bf16_t* Wr, const bf16_t* X, bf16_t* dX,
                           float* dW, void* ws, hipStream_t st);
size_t router_dw_workspace_bytes(int T, int d, int E);

// fp32 path (plain FMA kernels; every GEMM of the layer in float)
hipError_t gemm1_fwd_f32(const GemmShape& s, const int* offsets, const float* X, const float* W1, const float* W3,
                         float* ab, float* h, hipStream_t st);
hipError_t gemm2_fwd_f32(const GemmShape& s, const int* offsets, const float* H, const float* W2, float* Y,
                         hipStream_t st);
hipError_t dgrad2_f32(const GemmShape& s, const int* offsets, const float* dY, const float* W2, const float* ab,
                      float* dab, hipStream_t st);
hipError_t wgrad2_f32(const GemmShape& s, const int* offsets, const float* H, const float* dY, float* dW2,
                      hipStream_t st);
hipError_t dgrad1_f32(const GemmShape& s, const int* offsets, const float* dab, const float* W1, const float* W3,
                      float* dX, hipStream_t st);
hipError_t wgrad1_f32(const GemmShape& s, const int* offsets, const float* X, const float* dab, float* dW1,
                      float* dW3, hipStream_t st);
hipError_t router_fwd_f32(int T, int d, int E, const float* X, const float* Wr, const float* bias, float* L,
                          hipStream_t st);
hipError_t router_dx_f32(int T, int d, int E, const float* dL, const float* Wr, float* dX, hipStream_t st);
hipError_t router_dw_f32(int T, int d, int E, const float* dL, const float* X, float* dW, hipStream_t st);

}  // namespace moe
