// C ABI of the SiLU-gated RMSNorm library: argument checking, then launches.
// Every rule enforced here is stated in include/gated_rmsnorm.h.
#include "gated_rmsnorm.h"
#include "launch.h"

#include <cmath>
#include <cstdlib>

namespace {

constexpr int32_t kSupportedD = 128;
constexpr size_t kRowBytes = kSupportedD * 2;  // one BF16 row

struct Range {
  const void* p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a.p);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(b.p);
  return pa < pb + b.n && pb < pa + a.n;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Launch-shape cap from the environment (0 = no cap).
int env_max_wg() {
  const char* s = std::getenv("GATED_RMSNORM_MAX_WG");
  if (s == nullptr || *s == '\0') return 0;
  char* end = nullptr;
  const long v = std::strtol(s, &end, 10);
  if (end == s || v <= 0 || v > (1L << 30)) return 0;
  return static_cast<int>(v);
}

grn_status check_common(int64_t rows, int32_t D, int32_t dtype) {
  if (D != kSupportedD || rows < 0 || rows > GRN_MAX_ROWS) return GRN_ERR_SHAPE;
  if (dtype != GRN_DTYPE_BF16) return GRN_ERR_DTYPE;
  return GRN_OK;
}

grn_status check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.0f) return GRN_ERR_EPS;
  return GRN_OK;
}

size_t workspace_need(int64_t rows) {
  return rows > 0 ? grn::bwd_layout(rows).bytes : 0;
}

// Pointer rules shared by every entry point.  `acts` are [rows, D] BF16
// activations (inputs first, then outputs); `n_in` of them are inputs.
grn_status check_buffers(int64_t rows, const void* const* acts, int n_acts,
                         int n_in, const void* w, const void* ws,
                         size_t ws_need, const void* dw, size_t dw_bytes) {
  const size_t act_bytes = static_cast<size_t>(rows) * kRowBytes;
  if (w == nullptr) return GRN_ERR_NULL;
  if (rows > 0)
    for (int k = 0; k < n_acts; ++k)
      if (acts[k] == nullptr) return GRN_ERR_NULL;
  if (dw_bytes > 0 && dw == nullptr) return GRN_ERR_NULL;
  if (ws_need > 0 && ws == nullptr) return GRN_ERR_WORKSPACE;

  if (!aligned(w, 16)) return GRN_ERR_ALIGN;
  for (int k = 0; k < n_acts; ++k)
    if (!aligned(acts[k], 16)) return GRN_ERR_ALIGN;
  if (ws_need > 0 && !aligned(ws, 16)) return GRN_ERR_ALIGN;
  if (dw_bytes > 0 && !aligned(dw, dw_bytes / kSupportedD)) return GRN_ERR_ALIGN;

  // Outputs: activations n_in.., dw, and the workspace (written as scratch).
  Range outs[8];
  int n_out = 0;
  for (int k = n_in; k < n_acts; ++k) outs[n_out++] = Range{acts[k], act_bytes};
  if (dw_bytes > 0) outs[n_out++] = Range{dw, dw_bytes};
  if (ws_need > 0) outs[n_out++] = Range{ws, ws_need};
  Range ins[8];
  int n_ins = 0;
  for (int k = 0; k < n_in; ++k) ins[n_ins++] = Range{acts[k], act_bytes};
  ins[n_ins++] = Range{w, kRowBytes};
  for (int a = 0; a < n_out; ++a) {
    for (int b = 0; b < n_ins; ++b)
      if (overlap(outs[a], ins[b])) return GRN_ERR_ALIAS;
    for (int b = a + 1; b < n_out; ++b)
      if (overlap(outs[a], outs[b])) return GRN_ERR_ALIAS;
  }
  return GRN_OK;
}

grn_status hip_status(hipError_t e) { return e == hipSuccess ? GRN_OK : GRN_ERR_HIP; }

}  // namespace

extern "C" {

size_t gated_rmsnorm_workspace_bytes(int64_t rows, int32_t D) {
  if (D != kSupportedD || rows <= 0 || rows > GRN_MAX_ROWS) return 0;
  return workspace_need(rows);
}

int32_t gated_rmsnorm_chunk_rows(void) { return grn::kChunkRows; }

size_t gated_rmsnorm_workspace_init_bytes(void) { return grn::kCounterBytes; }

grn_status gated_rmsnorm_fwd(const void* x, const void* g, const void* w,
                             void* y, int64_t rows, int32_t D, float eps,
                             int32_t dtype, void* stream) {
  grn_status st = check_common(rows, D, dtype);
  if (st != GRN_OK) return st;
  if ((st = check_eps(eps)) != GRN_OK) return st;
  const void* acts[3] = {x, g, y};
  st = check_buffers(rows, acts, 3, 2, w, nullptr, 0, nullptr, 0);
  if (st != GRN_OK) return st;
  return hip_status(grn::launch_fwd(x, g, w, y, rows, eps, env_max_wg(),
                                    static_cast<hipStream_t>(stream)));
}

grn_status gated_rmsnorm_bwd(const void* x, const void* g, const void* w,
                             const void* dy, void* dx, void* dg, void* dw,
                             void* workspace, size_t workspace_bytes,
                             int64_t rows, int32_t D, float eps,
                             int32_t dtype, int32_t dw_fp32, void* stream) {
  grn_status st = check_common(rows, D, dtype);
  if (st != GRN_OK) return st;
  if (dw_fp32 != 0 && dw_fp32 != 1) return GRN_ERR_DTYPE;
  if ((st = check_eps(eps)) != GRN_OK) return st;
  const size_t need = workspace_need(rows);
  if (workspace_bytes < need) return GRN_ERR_WORKSPACE;
  const void* acts[5] = {x, g, dy, dx, dg};
  st = check_buffers(rows, acts, 5, 3, w, workspace, need, dw,
                     kSupportedD * (dw_fp32 ? 4 : 2));
  if (st != GRN_OK) return st;
  return hip_status(grn::launch_bwd(x, g, w, dy, dx, dg, dw, dw_fp32, workspace,
                                    rows, eps, env_max_wg(),
                                    static_cast<hipStream_t>(stream)));
}

grn_status gated_rmsnorm_ckpt_step(const void* x, const void* g,
                                   const void* w, const void* dy, void* y,
                                   void* dx, void* dg, void* dw,
                                   void* workspace, size_t workspace_bytes,
                                   int64_t rows, int32_t D, float eps,
                                   int32_t dtype, int32_t dw_fp32,
                                   void* stream) {
  grn_status st = check_common(rows, D, dtype);
  if (st != GRN_OK) return st;
  if (dw_fp32 != 0 && dw_fp32 != 1) return GRN_ERR_DTYPE;
  if ((st = check_eps(eps)) != GRN_OK) return st;
  const size_t need = workspace_need(rows);
  if (workspace_bytes < need) return GRN_ERR_WORKSPACE;
  const void* acts[6] = {x, g, dy, y, dx, dg};
  st = check_buffers(rows, acts, 6, 3, w, workspace, need, dw,
                     kSupportedD * (dw_fp32 ? 4 : 2));
  if (st != GRN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int max_wg = env_max_wg();
  for (int pass = 0; pass < 2; ++pass) {
    if (grn::launch_fwd(x, g, w, y, rows, eps, max_wg, s) != hipSuccess)
      return GRN_ERR_HIP;
  }
  return hip_status(grn::launch_bwd(x, g, w, dy, dx, dg, dw, dw_fp32, workspace,
                                    rows, eps, max_wg, s));
}

grn_status gated_rmsnorm_workspace_init(void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (workspace == nullptr) return GRN_ERR_NULL;
  if (workspace_bytes < grn::kCounterBytes) return GRN_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return GRN_ERR_ALIGN;
  return hip_status(grn::launch_counters_zero(workspace,
                                              static_cast<hipStream_t>(stream)));
}

const char* gated_rmsnorm_status_string(int32_t status) {
  switch (status) {
    case GRN_OK: return "GRN_OK: success";
    case GRN_ERR_NULL: return "GRN_ERR_NULL: a required pointer is NULL";
    case GRN_ERR_SHAPE: return "GRN_ERR_SHAPE: D must be 128 and 0 <= rows <= 2^31-1";
    case GRN_ERR_DTYPE: return "GRN_ERR_DTYPE: dtype must be BF16 and dw_fp32 0 or 1";
    case GRN_ERR_ALIGN: return "GRN_ERR_ALIGN: a pointer is misaligned";
    case GRN_ERR_ALIAS: return "GRN_ERR_ALIAS: an output overlaps another buffer";
    case GRN_ERR_WORKSPACE: return "GRN_ERR_WORKSPACE: workspace missing or too small";
    case GRN_ERR_EPS: return "GRN_ERR_EPS: eps must be finite and >= 0";
    case GRN_ERR_HIP: return "GRN_ERR_HIP: the HIP runtime reported a launch error";
    default: return "unknown gated_rmsnorm status";
  }
}

}  // extern "C"
