// C ABI of the SiLU-gated RMSNorm library: argument checking, then launches.
// Every rule enforced here is stated in include/gated_rmsnorm.h.
#include "gated_rmsnorm.h"
#include "launch.h"

#include <cmath>
#include <cstdlib>
#include <mutex>

namespace {

bool supported_d(int32_t D) { return D == 64 || D == 128 || D == 256; }

bool supported_dtype(int32_t dtype) {
  return dtype == GRN_DTYPE_BF16 || dtype == GRN_DTYPE_F16 || dtype == GRN_DTYPE_F32;
}

// Bytes per element of a supported dtype.
int64_t elem_bytes(int32_t dtype) { return dtype == GRN_DTYPE_F32 ? 4 : 2; }

// A set of `rows` rows of `width` bytes, `pitch` bytes apart, from `p`.
struct Rows {
  const void* p;
  int64_t rows;
  int64_t pitch;
  int64_t width;
};

uintptr_t extent(const Rows& a) {
  return a.rows <= 0 ? 0 : (uintptr_t)((a.rows - 1) * a.pitch + a.width);
}

// True if two row sets share a byte.  Exact when the pitches are equal
// (rows interleaved in one buffer, e.g. two halves of a fused projection, do
// not overlap); conservative (address ranges) otherwise.
bool overlap(const Rows& a, const Rows& b) {
  const uintptr_t ea = extent(a), eb = extent(b);
  if (a.p == nullptr || b.p == nullptr || ea == 0 || eb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a.p);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(b.p);
  if (!(pa < pb + eb && pb < pa + ea)) return false;
  if (a.pitch != b.pitch || a.rows <= 1 || b.rows <= 1) return true;
  const uintptr_t pitch = (uintptr_t)a.pitch;
  const uintptr_t lo = pa < pb ? pa : pb;
  const uintptr_t delta = ((pa < pb ? pb : pa) - lo) % pitch;
  const uintptr_t w_lo = (pa < pb ? a.width : b.width);   // row width at lo
  const uintptr_t w_hi = (pa < pb ? b.width : a.width);
  // rows of the later set start `delta` bytes into each pitch of the earlier
  return !(delta >= w_lo && delta + w_hi <= pitch);
}

Rows plain(const void* p, size_t bytes) {
  return Rows{p, bytes > 0 ? 1 : 0, (int64_t)bytes, (int64_t)bytes};
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

// Test knob: a set, non-empty GATED_RMSNORM_CKPT_SKIP_FIRST_FWD (other than
// "0") makes the checkpointed step skip its first forward, so that y comes
// from the recomputed forward alone (inside the backward's launch where the
// step fuses them).
bool env_skip_first_fwd() {
  const char* s = std::getenv("GATED_RMSNORM_CKPT_SKIP_FIRST_FWD");
  return s != nullptr && *s != '\0' && !(s[0] == '0' && s[1] == '\0');
}

grn_status check_common(int64_t rows, int32_t D, int32_t dtype) {
  if (!supported_d(D) || rows < 0 || rows > GRN_MAX_ROWS) return GRN_ERR_SHAPE;
  if (!supported_dtype(dtype)) return GRN_ERR_DTYPE;
  return GRN_OK;
}

grn_status check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.0f) return GRN_ERR_EPS;
  return GRN_OK;
}

// A row stride (elements) is at least D, at most kMaxStride, and keeps every
// row 16-byte aligned.
grn_status check_stride(int64_t stride, int32_t D, int64_t esize) {
  if (stride < D || stride > grn::kMaxStride) return GRN_ERR_SHAPE;
  if ((stride * esize) % 16 != 0) return GRN_ERR_ALIGN;
  return GRN_OK;
}

// Workspace bytes of a call (esize > 0), or the most any element type needs
// (esize = 0).
size_t workspace_need(int64_t rows, int32_t D, int32_t esize) {
  return rows > 0 ? grn::bwd_layout(rows, D, esize).bytes : 0;
}

struct Act {
  const void* p;
  int64_t stride;  // elements
};

// Pointer rules shared by every entry point.  `acts` are [rows, D]
// activations of `esize`-byte elements (inputs first, then outputs); `n_in`
// of them are inputs.  w is [D] of the same type; dw is `dw_bytes` bytes.
grn_status check_buffers(int64_t rows, int32_t D, int64_t esize, const Act* acts,
                         int n_acts, int n_in, const void* w, const void* ws,
                         size_t ws_need, const void* dw, size_t dw_bytes) {
  if (w == nullptr) return GRN_ERR_NULL;
  if (rows > 0)
    for (int k = 0; k < n_acts; ++k)
      if (acts[k].p == nullptr) return GRN_ERR_NULL;
  if (dw_bytes > 0 && dw == nullptr) return GRN_ERR_NULL;
  if (ws_need > 0 && ws == nullptr) return GRN_ERR_WORKSPACE;

  for (int k = 0; k < n_acts; ++k) {
    const grn_status st = check_stride(acts[k].stride, D, esize);
    if (st != GRN_OK) return st;
  }
  if (!aligned(w, 16)) return GRN_ERR_ALIGN;
  for (int k = 0; k < n_acts; ++k)
    if (!aligned(acts[k].p, 16)) return GRN_ERR_ALIGN;
  if (ws_need > 0 && !aligned(ws, 16)) return GRN_ERR_ALIGN;
  if (dw_bytes > 0 && !aligned(dw, dw_bytes / D)) return GRN_ERR_ALIGN;

  // Outputs: activations n_in.., dw, and the workspace (written as scratch).
  const int64_t row_bytes = D * esize;
  Rows outs[8];
  int n_out = 0;
  for (int k = n_in; k < n_acts; ++k)
    outs[n_out++] = Rows{acts[k].p, rows, acts[k].stride * esize, row_bytes};
  if (dw_bytes > 0) outs[n_out++] = plain(dw, dw_bytes);
  if (ws_need > 0) outs[n_out++] = plain(ws, ws_need);
  Rows ins[8];
  int n_ins = 0;
  for (int k = 0; k < n_in; ++k)
    ins[n_ins++] = Rows{acts[k].p, rows, acts[k].stride * esize, row_bytes};
  ins[n_ins++] = plain(w, (size_t)row_bytes);
  for (int a = 0; a < n_out; ++a) {
    for (int b = 0; b < n_ins; ++b)
      if (overlap(outs[a], ins[b])) return GRN_ERR_ALIAS;
    for (int b = a + 1; b < n_out; ++b)
      if (overlap(outs[a], outs[b])) return GRN_ERR_ALIAS;
  }
  return GRN_OK;
}

// Bytes of dw: FP32 if asked for, else the input type.
size_t dw_size(int32_t D, int32_t dtype, int32_t dw_fp32) {
  return (size_t)D * (dw_fp32 ? 4 : elem_bytes(dtype));
}

grn_status hip_status(hipError_t e) { return e == hipSuccess ? GRN_OK : GRN_ERR_HIP; }

// ---------------------------------------------------------------------------
// Scratch of gated_rmsnorm_bwd_noalloc: the backward's workspace (arrival
// counters, then the dw partials) in a static device array, one copy per
// GPU, held from the library's loading until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: the device
// address is fetched once per device with hipGetSymbolAddress and only that
// address is ever handed to a kernel.
static_assert(GRN_NOALLOC_SCRATCH_BYTES % 256 == 0, "a whole number of 256-byte blocks");
static __device__ __align__(256) unsigned char scratch[GRN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;                 // device address of this device's copy
  hipError_t err = hipErrorNotInitialized;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch, set up on this device's
// first call: hipGetSymbolAddress, then the arrival counters zeroed by a
// small kernel enqueued on `s` (no memset: the call may be under graph
// capture).  Every completed backward leaves the counters at zero again.
hipError_t scratch_for(int dev, hipStream_t s, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p == nullptr) e = hipErrorInvalidSymbol;
    if (e == hipSuccess) e = grn::launch_counters_zero(p, s);
    slot.ptr = e == hipSuccess ? p : nullptr;
    slot.err = e;
  });
  *out = slot.ptr;
  return slot.err;
}

}  // namespace

extern "C" {

size_t gated_rmsnorm_workspace_bytes(int64_t rows, int32_t D) {
  if (!supported_d(D) || rows <= 0 || rows > GRN_MAX_ROWS) return 0;
  return workspace_need(rows, D, 0);
}

int32_t gated_rmsnorm_chunk_rows(int64_t rows, int32_t D, int32_t dtype) {
  if (rows <= 0 || !supported_d(D) || !supported_dtype(dtype)) return 0;
  return grn::chunk_rows_for(D * (int32_t)elem_bytes(dtype));
}

size_t gated_rmsnorm_workspace_init_bytes(void) { return grn::kCounterBytes; }

grn_status gated_rmsnorm_fwd_strided(const void* x, int64_t x_stride,
                                     const void* g, int64_t g_stride,
                                     const void* w, void* y, int64_t y_stride,
                                     int64_t rows, int32_t D, float eps,
                                     int32_t dtype, void* stream) {
  grn_status st = check_common(rows, D, dtype);
  if (st != GRN_OK) return st;
  if ((st = check_eps(eps)) != GRN_OK) return st;
  const Act acts[3] = {{x, x_stride}, {g, g_stride}, {y, y_stride}};
  st = check_buffers(rows, D, elem_bytes(dtype), acts, 3, 2, w, nullptr, 0, nullptr, 0);
  if (st != GRN_OK) return st;
  grn::RowStrides rs;
  rs.x = x_stride;
  rs.g = g_stride;
  rs.y = y_stride;
  return hip_status(grn::launch_fwd(x, g, w, y, rs, rows, D, dtype, eps, env_max_wg(),
                                    static_cast<hipStream_t>(stream)));
}

grn_status gated_rmsnorm_fwd(const void* x, const void* g, const void* w,
                             void* y, int64_t rows, int32_t D, float eps,
                             int32_t dtype, void* stream) {
  return gated_rmsnorm_fwd_strided(x, D, g, D, w, y, D, rows, D, eps, dtype, stream);
}

grn_status gated_rmsnorm_bwd_strided(const void* x, int64_t x_stride,
                                     const void* g, int64_t g_stride,
                                     const void* w, const void* dy,
                                     int64_t dy_stride, void* dx,
                                     int64_t dx_stride, void* dg,
                                     int64_t dg_stride, void* dw,
                                     void* workspace, size_t workspace_bytes,
                                     int64_t rows, int32_t D, float eps,
                                     int32_t dtype, int32_t dw_fp32,
                                     int32_t deterministic, void* stream) {
  grn_status st = check_common(rows, D, dtype);
  if (st != GRN_OK) return st;
  if (dw_fp32 != 0 && dw_fp32 != 1) return GRN_ERR_DTYPE;
  if (deterministic != 0 && deterministic != 1) return GRN_ERR_ARG;
  if ((st = check_eps(eps)) != GRN_OK) return st;
  const size_t need = workspace_need(rows, D, (int32_t)elem_bytes(dtype));
  if (workspace_bytes < need) return GRN_ERR_WORKSPACE;
  const Act acts[5] = {{x, x_stride}, {g, g_stride}, {dy, dy_stride},
                       {dx, dx_stride}, {dg, dg_stride}};
  st = check_buffers(rows, D, elem_bytes(dtype), acts, 5, 3, w, workspace, need, dw,
                     dw_size(D, dtype, dw_fp32));
  if (st != GRN_OK) return st;
  grn::RowStrides rs;
  rs.x = x_stride;
  rs.g = g_stride;
  rs.dy = dy_stride;
  rs.dx = dx_stride;
  rs.dg = dg_stride;
  return hip_status(grn::launch_bwd(x, g, w, dy, dx, dg, dw, dw_fp32, deterministic,
                                    workspace, rs, rows, D, dtype, eps, env_max_wg(),
                                    static_cast<hipStream_t>(stream)));
}

grn_status gated_rmsnorm_bwd(const void* x, const void* g, const void* w,
                             const void* dy, void* dx, void* dg, void* dw,
                             void* workspace, size_t workspace_bytes,
                             int64_t rows, int32_t D, float eps,
                             int32_t dtype, int32_t dw_fp32, void* stream) {
  return gated_rmsnorm_bwd_strided(x, D, g, D, w, dy, D, dx, D, dg, D, dw,
                                   workspace, workspace_bytes, rows, D, eps,
                                   dtype, dw_fp32, 1, stream);
}

grn_status gated_rmsnorm_bwd_noalloc(const void* x, const void* g, const void* w,
                                     const void* dy, void* dx, void* dg, void* dw,
                                     int64_t rows, int32_t D, float eps, int32_t dtype,
                                     int32_t dw_fp32, void* stream) {
  grn_status st = check_common(rows, D, dtype);
  if (st != GRN_OK) return st;
  if (dw_fp32 != 0 && dw_fp32 != 1) return GRN_ERR_DTYPE;
  if ((st = check_eps(eps)) != GRN_OK) return st;
  const size_t need = workspace_need(rows, D, (int32_t)elem_bytes(dtype));
  if (need > (size_t)GRN_NOALLOC_SCRATCH_BYTES) return GRN_ERR_SCRATCH;
  const Act acts[5] = {{x, D}, {g, D}, {dy, D}, {dx, D}, {dg, D}};
  st = check_buffers(rows, D, elem_bytes(dtype), acts, 5, 3, w, nullptr, 0, dw,
                     dw_size(D, dtype, dw_fp32));
  if (st != GRN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GRN_ERR_HIP;
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return GRN_ERR_HIP;
    if ((int)sdev != dev) return GRN_ERR_ARG;
  }
  void* ws = nullptr;
  if (scratch_for(dev, s, &ws) != hipSuccess) return GRN_ERR_HIP;
  grn::RowStrides rs;
  rs.x = rs.g = rs.dy = rs.dx = rs.dg = D;
  return hip_status(grn::launch_bwd(x, g, w, dy, dx, dg, dw, dw_fp32, 1, ws, rs, rows, D,
                                    dtype, eps, env_max_wg(), s));
}

grn_status gated_rmsnorm_ckpt_step_strided(
    const void* x, int64_t x_stride, const void* g, int64_t g_stride,
    const void* w, const void* dy, int64_t dy_stride, void* y, int64_t y_stride,
    void* dx, int64_t dx_stride, void* dg, int64_t dg_stride, void* dw,
    void* workspace, size_t workspace_bytes, int64_t rows, int32_t D,
    float eps, int32_t dtype, int32_t dw_fp32, int32_t deterministic,
    void* stream) {
  grn_status st = check_common(rows, D, dtype);
  if (st != GRN_OK) return st;
  if (dw_fp32 != 0 && dw_fp32 != 1) return GRN_ERR_DTYPE;
  if (deterministic != 0 && deterministic != 1) return GRN_ERR_ARG;
  if ((st = check_eps(eps)) != GRN_OK) return st;
  const size_t need = workspace_need(rows, D, (int32_t)elem_bytes(dtype));
  if (workspace_bytes < need) return GRN_ERR_WORKSPACE;
  const Act acts[6] = {{x, x_stride},   {g, g_stride},   {dy, dy_stride},
                       {y, y_stride},   {dx, dx_stride}, {dg, dg_stride}};
  st = check_buffers(rows, D, elem_bytes(dtype), acts, 6, 3, w, workspace, need, dw,
                     dw_size(D, dtype, dw_fp32));
  if (st != GRN_OK) return st;
  grn::RowStrides rs;
  rs.x = x_stride;
  rs.g = g_stride;
  rs.y = y_stride;
  rs.dy = dy_stride;
  rs.dx = dx_stride;
  rs.dg = dg_stride;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int max_wg = env_max_wg();
  // Forward, then the recomputed forward and the backward: for small
  // tensors the recomputed forward runs inside the backward's launch
  // (grn::ckpt_fuses_forward), otherwise as a launch of its own.
  const bool fuse = grn::ckpt_fuses_forward(rows, D, dtype, deterministic);
  for (int pass = env_skip_first_fwd() ? 1 : 0; pass < (fuse ? 1 : 2); ++pass) {
    if (grn::launch_fwd(x, g, w, y, rs, rows, D, dtype, eps, max_wg, s) != hipSuccess)
      return GRN_ERR_HIP;
  }
  return hip_status(grn::launch_bwd(x, g, w, dy, dx, dg, dw, dw_fp32, deterministic,
                                    workspace, rs, rows, D, dtype, eps, max_wg, s,
                                    fuse ? y : nullptr));
}

grn_status gated_rmsnorm_ckpt_step(const void* x, const void* g,
                                   const void* w, const void* dy, void* y,
                                   void* dx, void* dg, void* dw,
                                   void* workspace, size_t workspace_bytes,
                                   int64_t rows, int32_t D, float eps,
                                   int32_t dtype, int32_t dw_fp32,
                                   void* stream) {
  return gated_rmsnorm_ckpt_step_strided(x, D, g, D, w, dy, D, y, D, dx, D, dg, D,
                                         dw, workspace, workspace_bytes, rows, D,
                                         eps, dtype, dw_fp32, 1, stream);
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
    case GRN_ERR_SHAPE: return "GRN_ERR_SHAPE: D must be 64, 128 or 256, 0 <= rows <= 2^31-1, and D <= stride <= 2^24";
    case GRN_ERR_DTYPE: return "GRN_ERR_DTYPE: dtype must be BF16, FP16 or FP32 and dw_fp32 0 or 1";
    case GRN_ERR_ALIGN: return "GRN_ERR_ALIGN: a pointer or row stride is not 16-byte aligned";
    case GRN_ERR_ALIAS: return "GRN_ERR_ALIAS: an output overlaps another buffer";
    case GRN_ERR_WORKSPACE: return "GRN_ERR_WORKSPACE: workspace missing or too small";
    case GRN_ERR_EPS: return "GRN_ERR_EPS: eps must be finite and >= 0";
    case GRN_ERR_HIP: return "GRN_ERR_HIP: the HIP runtime reported a launch error";
    case GRN_ERR_ARG: return "GRN_ERR_ARG: a flag argument is not 0 or 1, or the stream is not on the current device";
    case GRN_ERR_SCRATCH: return "GRN_ERR_SCRATCH: the call needs more workspace than the library's static scratch holds (GRN_NOALLOC_SCRATCH_BYTES; use gated_rmsnorm_bwd with a workspace)";
    default: return "unknown gated_rmsnorm status";
  }
}

}  // extern "C"
