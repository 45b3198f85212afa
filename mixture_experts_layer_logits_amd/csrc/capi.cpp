// C-ABI entry points of libmoe_mi355x.so: host-side argument checks, dtype dispatch and
// kernel launches on the caller's stream.  Nothing here allocates, synchronises or reads
// device memory; every routing quantity stays on the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "../../include/moe.h"
#include "gemm.h"
#include "mx.h"
#include "route.h"

namespace moe {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0: not yet read
std::mutex g_state_mu;                     // guards the two maps below
std::map<std::tuple<int, const void*, int, size_t>, int> g_occupancy;
std::map<std::string, std::string> g_env;  // names read so far; "\x01" marks an unset name

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  return dev;
}
}  // namespace

int device_cu_count() {
  const int dev = current_device();
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {  // every thread that races here reads the same attribute
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int kernel_occupancy(const void* kern, int threads, size_t dyn_lds) {
  const auto key = std::make_tuple(current_device(), kern, threads, dyn_lds);
  {
    std::lock_guard<std::mutex> lk(g_state_mu);
    auto it = g_occupancy.find(key);
    if (it != g_occupancy.end()) return it->second;
  }
  int o = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, threads, dyn_lds) != hipSuccess || o < 1) o = 1;
  std::lock_guard<std::mutex> lk(g_state_mu);
  return g_occupancy.emplace(key, o).first->second;
}

const char* tuning_env(const char* name) {
  std::lock_guard<std::mutex> lk(g_state_mu);
  auto it = g_env.find(name);
  if (it == g_env.end()) {
    const char* v = std::getenv(name);
    it = g_env.emplace(name, v ? std::string(v) : std::string("\x01")).first;
  }
  return it->second == "\x01" ? nullptr : it->second.c_str();  // map nodes never move
}

}  // namespace moe

using namespace moe;

namespace {

inline hipStream_t S(void* st) { return static_cast<hipStream_t>(st); }

inline moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(const moe_shape* s) { return s->act == MOE_F32 ? 4 : 2; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ENULL;
  if (s->T < 0 || s->d <= 0 || s->f <= 0 || s->E < 1 || s->E > kMaxExperts) return MOE_EINVAL;
  if (s->k < 1 || s->k > s->E || s->k > kMaxTopK) return MOE_EINVAL;
  if ((int64_t)s->T * s->k >= ((int64_t)1 << 31)) return MOE_EINVAL;
  if (s->d % 64 != 0 || s->f % 64 != 0) return MOE_EINVAL;
  if (s->act != MOE_F32 && s->act != MOE_BF16) return MOE_EUNSUPPORTED;
  if (s->gemm == MOE_F32 && s->act != MOE_F32) return MOE_EUNSUPPORTED;
  if ((s->gemm == MOE_BF16 || s->gemm == MOE_MXFP8) && s->act != MOE_BF16) return MOE_EUNSUPPORTED;
  if (s->gemm != MOE_F32 && s->gemm != MOE_BF16 && s->gemm != MOE_MXFP8) return MOE_EUNSUPPORTED;
  if (s->gemm == MOE_MXFP8 && (s->d % 128 != 0 || s->f % 128 != 0)) return MOE_EINVAL;
  if (s->mx_scope < 0 || (s->mx_scope & ~MOE_MX_ALL) != 0) return MOE_EINVAL;
  if (s->gemm != MOE_MXFP8 && s->mx_scope != 0) return MOE_EINVAL;
  return MOE_OK;
}

// Does the expert GEMM `bit` (MOE_MX_*) take MXFP8 operands under this shape?
bool mx_on(const moe_shape* s, int bit) {
  if (s->gemm != MOE_MXFP8) return false;
  const int scope = s->mx_scope ? s->mx_scope : MOE_MX_DEFAULT;
  return (scope & bit) != 0;
}

// every pointer non-null and 16-byte aligned
moe_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return MOE_ENULL;
    if (!aligned16(p)) return MOE_EALIGN;
  }
  return MOE_OK;
}

// buffers with T or T*k rows: may be NULL when T == 0 (nothing is read or written)
moe_status check_rows(const moe_shape* s, std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) {
      if (s->T == 0) continue;
      return MOE_ENULL;
    }
    if (!aligned16(p)) return MOE_EALIGN;
  }
  return MOE_OK;
}

bool rows_ok(const moe_shape* s, const void* p) { return p || s->T == 0; }

#define MOE_TRY(expr)                 \
  do {                                \
    moe_status _st = (expr);          \
    if (_st != MOE_OK) return _st;    \
  } while (0)

GemmShape gshape(const moe_shape* s) { return GemmShape{s->T * s->k, s->d, s->f, s->E}; }

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid shape or argument";
    case MOE_ENULL: return "null pointer";
    case MOE_EALIGN: return "pointer not 16-byte aligned";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EUNSUPPORTED: return "unsupported dtype combination";
    case MOE_ELAUNCH: return "kernel launch failed";
    case MOE_ESCRATCH: return "shape too large for the allocation-free entry point's fixed scratch (4 MiB)";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  size_t b = route_workspace_bytes(s->T, s->E, s->k);
  if (s->act == MOE_BF16) {
    const size_t r = router_dw_workspace_bytes(s->T, s->d, s->E);
    if (r > b) b = r;
  }
  if (s->gemm == MOE_BF16 || s->gemm == MOE_MXFP8) {  // bf16 weight gradients (any GEMM outside the MXFP8 scope)
    const size_t w = wgrad_split_workspace_bytes(gshape(s));
    if (w > b) b = w;
  }
  if (s->gemm == MOE_MXFP8) {
    const size_t m = mx_workspace_bytes(s->T * s->k, s->d, s->f, s->E);
    if (m > b) b = m;
  }
  return ((b + 255) / 256) * 256 + 256;
}

moe_status moe_router_fwd(const moe_shape* s, const void* x, const void* Wr, const float* bias, float* logits,
                          void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({Wr}));
  MOE_TRY(check_rows(s, {x, logits}));
  if (s->T == 0) return MOE_OK;
  if (s->act == MOE_F32)
    return launched(router_fwd_f32(s->T, s->d, s->E, (const float*)x, (const float*)Wr, bias, logits, S(st)));
  return launched(router_fwd_bf16(s->T, s->d, s->E, (const bf16_t*)x, (const bf16_t*)Wr, bias, logits, S(st)));
}

moe_status moe_route(const moe_shape* s, const float* logits, int32_t* topk_idx, float* gates, int32_t* counts,
                     int32_t* offsets, int32_t* slot_row, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  if (!rows_ok(s, logits) || !rows_ok(s, topk_idx) || !rows_ok(s, gates) || !rows_ok(s, slot_row)) return MOE_ENULL;
  if (!counts || !offsets || !ws) return MOE_ENULL;
  if (ws_bytes < route_workspace_bytes(s->T, s->E, s->k)) return MOE_EWORKSPACE;
  return launched(route_topk(s->T, s->E, s->k, logits, topk_idx, gates, counts, offsets, slot_row, ws, S(st)));
}

moe_status moe_route_noalloc(const moe_shape* s, const float* logits, int32_t* topk_idx, float* gates,
                             int32_t* counts, int32_t* offsets, int32_t* slot_row, void* st) {
  MOE_TRY(check_shape(s));
  if (!rows_ok(s, logits) || !rows_ok(s, topk_idx) || !rows_ok(s, gates) || !rows_ok(s, slot_row)) return MOE_ENULL;
  if (!counts || !offsets) return MOE_ENULL;
  if (route_workspace_bytes(s->T, s->E, s->k) > kRouteScratchInts * sizeof(int32_t)) return MOE_ESCRATCH;
  int32_t* scr = nullptr;
  if (route_scratch_ptr(&scr) != hipSuccess) return MOE_ELAUNCH;
  return launched(route_topk(s->T, s->E, s->k, logits, topk_idx, gates, counts, offsets, slot_row, scr, S(st)));
}

moe_status moe_route_given(const moe_shape* s, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                           int32_t* slot_row, int32_t* dev_err, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  if (!rows_ok(s, topk_idx) || !rows_ok(s, slot_row)) return MOE_ENULL;
  if (!counts || !offsets || !dev_err || !ws) return MOE_ENULL;
  if (ws_bytes < route_workspace_bytes(s->T, s->E, s->k)) return MOE_EWORKSPACE;
  return launched(route_given(s->T, s->E, s->k, topk_idx, counts, offsets, slot_row, dev_err, ws, S(st)));
}

moe_status moe_permute(const moe_shape* s, const void* x, const int32_t* slot_row, int32_t* row_src, void* x_perm,
                       void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_rows(s, {x, x_perm}));
  if (!rows_ok(s, slot_row)) return MOE_ENULL;
  return launched(permute_rows(elem_bytes(s), s->T, s->d, s->k, x, slot_row, row_src, x_perm, S(st)));
}

moe_status moe_ffn_gemm1_fwd(const moe_shape* s, const void* x_perm, const void* W1, const void* W3,
                             const int32_t* offsets, void* ab, void* h, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({W1, W3}));
  MOE_TRY(check_rows(s, {x_perm, ab, h}));
  if (!offsets) return MOE_ENULL;
  const GemmShape g = gshape(s);
  switch (s->gemm == MOE_F32 ? 0 : mx_on(s, MOE_MX_GEMM1) ? 2 : 1) {
    case 0:
      return launched(gemm1_fwd_f32(g, offsets, (const float*)x_perm, (const float*)W1, (const float*)W3,
                                    (float*)ab, (float*)h, S(st)));
    case 1:
      return launched(gemm1_fwd_bf16(g, offsets, (const bf16_t*)x_perm, (const bf16_t*)W1, (const bf16_t*)W3,
                                     (bf16_t*)ab, (bf16_t*)h, S(st)));
    default:
      if (!ws) return MOE_ENULL;
      if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
      return launched(gemm1_fwd_mx(g, offsets, (const bf16_t*)x_perm, (const bf16_t*)W1, (const bf16_t*)W3,
                                   (bf16_t*)ab, (bf16_t*)h, ws, S(st)));
  }
}

moe_status moe_ffn_gemm2_fwd(const moe_shape* s, const void* h, const void* W2, const int32_t* offsets,
                             void* y_perm, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({W2}));
  MOE_TRY(check_rows(s, {h, y_perm}));
  if (!offsets) return MOE_ENULL;
  const GemmShape g = gshape(s);
  switch (s->gemm == MOE_F32 ? 0 : mx_on(s, MOE_MX_GEMM2) ? 2 : 1) {
    case 0:
      return launched(gemm2_fwd_f32(g, offsets, (const float*)h, (const float*)W2, (float*)y_perm, S(st)));
    case 1:
      return launched(gemm2_fwd_bf16(g, offsets, (const bf16_t*)h, (const bf16_t*)W2, (bf16_t*)y_perm, S(st)));
    default:
      if (!ws) return MOE_ENULL;
      if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
      return launched(gemm2_fwd_mx(g, offsets, (const bf16_t*)h, (const bf16_t*)W2, (bf16_t*)y_perm, ws, S(st)));
  }
}

moe_status moe_grouped_ffn_fwd(const moe_shape* s, const void* x_perm, const void* W1, const void* W3,
                               const void* W2, const int32_t* offsets, void* ab, void* h, void* y_perm, void* ws,
                               size_t ws_bytes, void* st) {
  MOE_TRY(moe_ffn_gemm1_fwd(s, x_perm, W1, W3, offsets, ab, h, ws, ws_bytes, st));
  return moe_ffn_gemm2_fwd(s, h, W2, offsets, y_perm, ws, ws_bytes, st);
}

moe_status moe_combine(const moe_shape* s, const void* y_perm, const float* gates, const int32_t* slot_row,
                       const void* y_add, void* y, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_rows(s, {y_perm, y}));
  if (!rows_ok(s, gates) || !rows_ok(s, slot_row)) return MOE_ENULL;
  if (y_add && !aligned16(y_add)) return MOE_EALIGN;
  return launched(combine_rows(elem_bytes(s), s->T, s->d, s->k, y_perm, gates, slot_row, y_add, y, S(st)));
}

moe_status moe_combine_bwd(const moe_shape* s, const void* dy, const void* y_perm, const float* gates,
                           const int32_t* slot_row, void* dy_perm, float* dgates, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_rows(s, {dy, y_perm, dy_perm}));
  if (!rows_ok(s, gates) || !rows_ok(s, slot_row) || !rows_ok(s, dgates)) return MOE_ENULL;
  return launched(
      combine_rows_bwd(elem_bytes(s), s->T, s->d, s->k, dy, y_perm, gates, slot_row, dy_perm, dgates, S(st)));
}

moe_status moe_ffn_dgrad2(const moe_shape* s, const void* dy_perm, const void* W2, const void* ab,
                          const int32_t* offsets, void* dab, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({W2}));
  MOE_TRY(check_rows(s, {dy_perm, ab, dab}));
  if (!offsets) return MOE_ENULL;
  const GemmShape g = gshape(s);
  switch (s->gemm == MOE_F32 ? 0 : mx_on(s, MOE_MX_DGRAD2) ? 2 : 1) {
    case 0:
      return launched(dgrad2_f32(g, offsets, (const float*)dy_perm, (const float*)W2, (const float*)ab, (float*)dab,
                                 S(st)));
    case 1:
      return launched(dgrad2_bf16(g, offsets, (const bf16_t*)dy_perm, (const bf16_t*)W2, (const bf16_t*)ab,
                                  (bf16_t*)dab, S(st)));
    default:
      if (!ws) return MOE_ENULL;
      if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
      return launched(dgrad2_mx(g, offsets, (const bf16_t*)dy_perm, (const bf16_t*)W2, (const bf16_t*)ab,
                                (bf16_t*)dab, ws, S(st)));
  }
}

moe_status moe_ffn_wgrad2(const moe_shape* s, const void* h, const void* dy_perm, const int32_t* offsets, void* dW2,
                          void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({dW2}));
  MOE_TRY(check_rows(s, {h, dy_perm}));
  if (!offsets) return MOE_ENULL;
  const GemmShape g = gshape(s);
  switch (s->gemm == MOE_F32 ? 0 : mx_on(s, MOE_MX_WGRAD2) ? 2 : 1) {
    case 0:
      return launched(wgrad2_f32(g, offsets, (const float*)h, (const float*)dy_perm, (float*)dW2, S(st)));
    case 1:
      if (g.E == 1 && ws_bytes < wgrad_split_workspace_bytes(g)) return MOE_EWORKSPACE;
      return launched(wgrad2_bf16(g, offsets, (const bf16_t*)h, (const bf16_t*)dy_perm, (bf16_t*)dW2, ws, S(st)));
    default:
      if (!ws) return MOE_ENULL;
      if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
      return launched(wgrad2_mx(g, offsets, (const bf16_t*)h, (const bf16_t*)dy_perm, (bf16_t*)dW2, ws, S(st)));
  }
}

moe_status moe_ffn_dgrad1(const moe_shape* s, const void* dab, const void* W1, const void* W3, const int32_t* offsets,
                          void* dx_perm, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({W1, W3}));
  MOE_TRY(check_rows(s, {dab, dx_perm}));
  if (!offsets) return MOE_ENULL;
  const GemmShape g = gshape(s);
  switch (s->gemm == MOE_F32 ? 0 : mx_on(s, MOE_MX_DGRAD1) ? 2 : 1) {
    case 0:
      return launched(dgrad1_f32(g, offsets, (const float*)dab, (const float*)W1, (const float*)W3, (float*)dx_perm,
                                 S(st)));
    case 1:
      return launched(dgrad1_bf16(g, offsets, (const bf16_t*)dab, (const bf16_t*)W1, (const bf16_t*)W3,
                                  (bf16_t*)dx_perm, S(st)));
    default:
      if (!ws) return MOE_ENULL;
      if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
      return launched(dgrad1_mx(g, offsets, (const bf16_t*)dab, (const bf16_t*)W1, (const bf16_t*)W3,
                                (bf16_t*)dx_perm, ws, S(st)));
  }
}

moe_status moe_ffn_wgrad1(const moe_shape* s, const void* x_perm, const void* dab, const int32_t* offsets, void* dW1,
                          void* dW3, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({dW1, dW3}));
  MOE_TRY(check_rows(s, {x_perm, dab}));
  if (!offsets) return MOE_ENULL;
  const GemmShape g = gshape(s);
  switch (s->gemm == MOE_F32 ? 0 : mx_on(s, MOE_MX_WGRAD1) ? 2 : 1) {
    case 0:
      return launched(wgrad1_f32(g, offsets, (const float*)x_perm, (const float*)dab, (float*)dW1, (float*)dW3,
                                 S(st)));
    case 1:
      if (g.E == 1 && ws_bytes < wgrad_split_workspace_bytes(g)) return MOE_EWORKSPACE;
      return launched(wgrad1_bf16(g, offsets, (const bf16_t*)x_perm, (const bf16_t*)dab, (bf16_t*)dW1,
                                  (bf16_t*)dW3, ws, S(st)));
    default:
      if (!ws) return MOE_ENULL;
      if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
      return launched(wgrad1_mx(g, offsets, (const bf16_t*)x_perm, (const bf16_t*)dab, (bf16_t*)dW1, (bf16_t*)dW3,
                                ws, S(st)));
  }
}

moe_status moe_grouped_ffn_bwd(const moe_shape* s, const void* dy_perm, const void* x_perm, const void* ab,
                               const void* h, const void* W1, const void* W3, const void* W2, const int32_t* offsets,
                               void* dab, void* dx_perm, void* dW1, void* dW3, void* dW2, void* ws, size_t ws_bytes,
                               void* st) {
  MOE_TRY(moe_ffn_dgrad2(s, dy_perm, W2, ab, offsets, dab, ws, ws_bytes, st));
  MOE_TRY(moe_ffn_wgrad2(s, h, dy_perm, offsets, dW2, ws, ws_bytes, st));
  MOE_TRY(moe_ffn_dgrad1(s, dab, W1, W3, offsets, dx_perm, ws, ws_bytes, st));
  return moe_ffn_wgrad1(s, x_perm, dab, offsets, dW1, dW3, ws, ws_bytes, st);
}

moe_status moe_route_bwd(const moe_shape* s, const float* dgates, const float* gates, const int32_t* topk_idx,
                         float* dlogits, void* st) {
  MOE_TRY(check_shape(s));
  if (!rows_ok(s, dgates) || !rows_ok(s, gates) || !rows_ok(s, topk_idx) || !rows_ok(s, dlogits)) return MOE_ENULL;
  if (s->T == 0) return MOE_OK;
  return launched(route_backward(s->T, s->E, s->k, dgates, gates, topk_idx, dlogits, S(st)));
}

moe_status moe_router_bwd(const moe_shape* s, const void* x, const void* Wr, const float* dlogits, void* dx_r,
                          float* dWr, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({Wr, dWr}));
  MOE_TRY(check_rows(s, {x}));
  if (dx_r && !aligned16(dx_r)) return MOE_EALIGN;
  if (!rows_ok(s, dlogits)) return MOE_ENULL;
  if (s->act == MOE_F32) {
    if (dx_r && s->T > 0 &&
        router_dx_f32(s->T, s->d, s->E, dlogits, (const float*)Wr, (float*)dx_r, S(st)) != hipSuccess)
      return MOE_ELAUNCH;
    return launched(router_dw_f32(s->T, s->d, s->E, dlogits, (const float*)x, dWr, S(st)));
  }
  if (!ws) return MOE_ENULL;
  if (ws_bytes < router_dw_workspace_bytes(s->T, s->d, s->E)) return MOE_EWORKSPACE;
  return launched(router_bwd_bf16(s->T, s->d, s->E, dlogits, (const bf16_t*)Wr, (const bf16_t*)x, (bf16_t*)dx_r, dWr,
                                  ws, S(st)));
}

moe_status moe_permute_bwd(const moe_shape* s, const void* dx_perm, const int32_t* slot_row, const void* dx_r,
                           const void* dx_add, void* dx, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_rows(s, {dx_perm, dx}));
  if (!rows_ok(s, slot_row)) return MOE_ENULL;
  if ((dx_r && !aligned16(dx_r)) || (dx_add && !aligned16(dx_add))) return MOE_EALIGN;
  return launched(
      unpermute_sum_rows(elem_bytes(s), s->T, s->d, s->k, dx_perm, slot_row, dx_r, dx_add, dx, S(st)));
}

moe_status moe_permute_bwd_router(const moe_shape* s, const void* dx_perm, const int32_t* slot_row,
                                  const int32_t* topk_idx, const float* dlogits, const void* Wr, const void* dx_add,
                                  void* dx, void* st) {
  MOE_TRY(check_shape(s));
  MOE_TRY(check_ptrs({Wr}));
  MOE_TRY(check_rows(s, {dx_perm, dx}));
  if (!rows_ok(s, slot_row) || !rows_ok(s, topk_idx) || !rows_ok(s, dlogits)) return MOE_ENULL;
  if (!aligned16(Wr) || (dx_add && !aligned16(dx_add))) return MOE_EALIGN;
  return launched(unpermute_router_rows(elem_bytes(s), s->T, s->d, s->k, s->E, dx_perm, slot_row, topk_idx, dlogits,
                                        Wr, dx_add, dx, S(st)));
}

moe_status moe_mx_quantize(int32_t rows, int32_t cols, int32_t axis, const int32_t* seg_offsets, int32_t nseg,
                           const void* src, uint8_t* q, uint8_t* scales, void* st) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_EINVAL;
  if (!src || !q || !scales) return MOE_ENULL;
  if (!aligned16(src) || !aligned16(q)) return MOE_EALIGN;
  if (axis == 0) return launched(mx_quantize_rows(rows, cols, (const bf16_t*)src, q, scales, S(st)));
  if (axis != 1 || nseg < 1 || nseg > kMaxExperts || !seg_offsets) return MOE_EINVAL;
  return launched(mx_quantize_cols_seg(rows, cols, seg_offsets, nseg, (const bf16_t*)src, q, scales, S(st)));
}

// ---------------------------------------------------------------------------------------
// MXFP8 dispatch and the expert GEMMs that take its quantised rows
// ---------------------------------------------------------------------------------------
size_t moe_mx_cols_ld(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return (size_t)s->T * s->k + (size_t)kMxSegPad * s->E;
}

moe_status moe_permute_mx(const moe_shape* s, const void* x, const int32_t* slot_row, const int32_t* offsets,
                          int32_t* row_src, uint8_t* q_rows, uint8_t* s_rows, uint8_t* q_cols, uint8_t* s_cols,
                          void* st) {
  MOE_TRY(check_shape(s));
  if (s->gemm != MOE_MXFP8) return MOE_EUNSUPPORTED;
  MOE_TRY(check_rows(s, {x, q_rows, s_rows, q_cols, s_cols}));
  if (!rows_ok(s, slot_row) || !rows_ok(s, row_src) || !offsets) return MOE_ENULL;
  if (s->T == 0) return MOE_OK;
  MOE_TRY(launched(row_src_rows(s->T, s->k, slot_row, row_src, S(st))));
  return launched(mx_dispatch(s->T * s->k, s->d, s->E, s->k, (const bf16_t*)x, row_src, offsets, nullptr, nullptr,
                              q_rows, s_rows, q_cols, s_cols, S(st)));
}

moe_status moe_combine_bwd_mx(const moe_shape* s, const void* dy, const void* y_perm, const float* gates,
                              const int32_t* slot_row, const int32_t* row_src, const int32_t* offsets, float* dgates,
                              uint8_t* q_rows, uint8_t* s_rows, uint8_t* q_cols, uint8_t* s_cols, void* st) {
  MOE_TRY(check_shape(s));
  if (s->gemm != MOE_MXFP8) return MOE_EUNSUPPORTED;
  MOE_TRY(check_rows(s, {dy, y_perm, q_rows, s_rows, q_cols, s_cols}));
  if (!rows_ok(s, gates) || !rows_ok(s, slot_row) || !rows_ok(s, row_src) || !rows_ok(s, dgates) || !offsets)
    return MOE_ENULL;
  if (s->T == 0) return MOE_OK;
  MOE_TRY(launched(dgates_rows(s->T, s->d, s->k, (const bf16_t*)dy, (const bf16_t*)y_perm, slot_row, dgates, S(st))));
  return launched(mx_dispatch(s->T * s->k, s->d, s->E, s->k, (const bf16_t*)dy, row_src, offsets, gates, slot_row,
                              q_rows, s_rows, q_cols, s_cols, S(st)));
}

moe_status moe_ffn_gemm1_fwd_mx(const moe_shape* s, const uint8_t* xq_rows, const uint8_t* xs_rows, const void* W1,
                                const void* W3, const int32_t* offsets, void* ab, void* h, void* ws, size_t ws_bytes,
                                void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_GEMM1)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({W1, W3}));
  MOE_TRY(check_rows(s, {xq_rows, xs_rows, ab, h}));
  if (!offsets || !ws) return MOE_ENULL;
  const GemmShape g = gshape(s);
  if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
  return launched(gemm1_fwd_mx(g, offsets, nullptr, (const bf16_t*)W1, (const bf16_t*)W3, (bf16_t*)ab, (bf16_t*)h, ws,
                               S(st), MxIn{xq_rows, xs_rows}));
}

moe_status moe_ffn_dgrad2_mx(const moe_shape* s, const uint8_t* dyq_rows, const uint8_t* dys_rows, const void* W2,
                             const void* ab, const int32_t* offsets, void* dab, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_DGRAD2)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({W2}));
  MOE_TRY(check_rows(s, {dyq_rows, dys_rows, ab, dab}));
  if (!offsets || !ws) return MOE_ENULL;
  const GemmShape g = gshape(s);
  if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
  return launched(dgrad2_mx(g, offsets, nullptr, (const bf16_t*)W2, (const bf16_t*)ab, (bf16_t*)dab, ws, S(st),
                            MxIn{dyq_rows, dys_rows}));
}

moe_status moe_ffn_wgrad2_mx(const moe_shape* s, const void* h, const uint8_t* dyq_cols, const uint8_t* dys_cols,
                             const int32_t* offsets, void* dW2, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_WGRAD2)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({dW2, dyq_cols, dys_cols}));
  MOE_TRY(check_rows(s, {h}));
  if (!offsets || !ws) return MOE_ENULL;
  const GemmShape g = gshape(s);
  if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
  return launched(wgrad2_mx(g, offsets, (const bf16_t*)h, nullptr, (bf16_t*)dW2, ws, S(st), MxIn{dyq_cols, dys_cols}));
}

moe_status moe_ffn_wgrad1_mx(const moe_shape* s, const uint8_t* xq_cols, const uint8_t* xs_cols, const void* dab,
                             const int32_t* offsets, void* dW1, void* dW3, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_WGRAD1)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({dW1, dW3, xq_cols, xs_cols}));
  MOE_TRY(check_rows(s, {dab}));
  if (!offsets || !ws) return MOE_ENULL;
  const GemmShape g = gshape(s);
  if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
  return launched(wgrad1_mx(g, offsets, nullptr, (const bf16_t*)dab, (bf16_t*)dW1, (bf16_t*)dW3, ws, S(st),
                            MxIn{xq_cols, xs_cols}));
}

void moe_tuning_reload(void) {
  std::lock_guard<std::mutex> lk(g_state_mu);
  g_env.clear();  // the next tuning_env call of each name reads the environment again
}

moe_status moe_ffn_gemm1_fwd_q(const moe_shape* s, const void* x_perm, const void* W1, const void* W3,
                               const int32_t* offsets, void* ab, void* h, uint8_t* hq_rows, uint8_t* hs_rows, void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_GEMM2) || mx_on(s, MOE_MX_GEMM1)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({W1, W3}));
  MOE_TRY(check_rows(s, {x_perm, ab, h, hq_rows, hs_rows}));
  if (!offsets) return MOE_ENULL;
  return launched(gemm1_fwd_bf16(gshape(s), offsets, (const bf16_t*)x_perm, (const bf16_t*)W1, (const bf16_t*)W3,
                                 (bf16_t*)ab, (bf16_t*)h, S(st), hq_rows, hs_rows));
}

moe_status moe_ffn_gemm2_fwd_mx(const moe_shape* s, const uint8_t* hq_rows, const uint8_t* hs_rows, const void* W2,
                                const int32_t* offsets, void* y_perm, void* ws, size_t ws_bytes, void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_GEMM2)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({W2}));
  MOE_TRY(check_rows(s, {hq_rows, hs_rows, y_perm}));
  if (!offsets || !ws) return MOE_ENULL;
  const GemmShape g = gshape(s);
  if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
  return launched(gemm2_fwd_mx(g, offsets, nullptr, (const bf16_t*)W2, (bf16_t*)y_perm, ws, S(st),
                               MxIn{hq_rows, hs_rows}));
}

moe_status moe_ffn_dgrad2_q(const moe_shape* s, const void* dy_perm, const void* W2, const void* ab,
                            const int32_t* offsets, void* dab, uint8_t* dabq_rows, uint8_t* dabs_rows, void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_DGRAD1) || mx_on(s, MOE_MX_DGRAD2)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({W2}));
  MOE_TRY(check_rows(s, {dy_perm, ab, dab, dabq_rows, dabs_rows}));
  if (!offsets) return MOE_ENULL;
  return launched(dgrad2_bf16(gshape(s), offsets, (const bf16_t*)dy_perm, (const bf16_t*)W2, (const bf16_t*)ab,
                              (bf16_t*)dab, S(st), dabq_rows, dabs_rows));
}

moe_status moe_ffn_dgrad1_mx(const moe_shape* s, const uint8_t* dabq_rows, const uint8_t* dabs_rows, const void* W1,
                             const void* W3, const int32_t* offsets, void* dx_perm, void* ws, size_t ws_bytes,
                             void* st) {
  MOE_TRY(check_shape(s));
  if (!mx_on(s, MOE_MX_DGRAD1)) return MOE_EUNSUPPORTED;
  MOE_TRY(check_ptrs({W1, W3}));
  MOE_TRY(check_rows(s, {dabq_rows, dabs_rows, dx_perm}));
  if (!offsets || !ws) return MOE_ENULL;
  const GemmShape g = gshape(s);
  if (ws_bytes < mx_workspace_bytes(g.R, g.d, g.f, g.E)) return MOE_EWORKSPACE;
  return launched(dgrad1_mx(g, offsets, nullptr, (const bf16_t*)W1, (const bf16_t*)W3, (bf16_t*)dx_perm, ws, S(st),
                            MxIn{dabq_rows, dabs_rows}));
}

}  // extern "C"
