// C ABI of the PT-DiT attention core: argument validation, workspace carving
// and kernel dispatch. Every check runs on the host before the first launch;
// nothing here allocates device memory or synchronises the caller's stream.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/ptdit.h"
#include "kernels.hpp"

using namespace ptdit;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
size_t esize(ptdit_dtype t) { return t == PTDIT_F32 ? 4 : 2; }
bool valid_dtype(ptdit_dtype t) { return t == PTDIT_BF16 || t == PTDIT_F32; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------------ trace
struct Trace {
  int cls = -1;
  int cap = 0;
  int count = 0;
  std::vector<hipEvent_t> start, stop;
} g_trace;

struct TraceScope {
  hipStream_t s;
  int slot = -1;
  TraceScope(int cls, hipStream_t st) : s(st) {
    if (g_trace.cls == cls && g_trace.count < g_trace.cap) {
      slot = g_trace.count++;
      (void)hipEventRecord(g_trace.start[slot], s);
    }
  }
  ~TraceScope() {
    if (slot >= 0) (void)hipEventRecord(g_trace.stop[slot], s);
  }
};

ptdit_status hip_status(hipError_t e) { return e == hipSuccess ? PTDIT_OK : PTDIT_ERR_HIP; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

int64_t floor_div(int64_t a, int64_t b) {  // b > 0
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// Do n batch blocks {a + i*sa, la bytes} and n blocks {b + j*sb, lb bytes}
// (i, j < n) share a byte? Exact for equal strides no shorter than the
// blocks (views of one fused [B][G][...] buffer interleave without
// overlapping); otherwise the whole extents are compared.
bool overlaps_strided(const void* a, int64_t sa, int64_t la, const void* b, int64_t sb, int64_t lb, int64_t n) {
  if (!a || !b || la <= 0 || lb <= 0 || n <= 0) return false;
  if (sa != sb || sa < la || sa < lb || n == 1)
    return overlaps(a, (size_t)((n - 1) * sa + la), b, (size_t)((n - 1) * sb + lb));
  const int64_t s = sa, d = (int64_t)((intptr_t)b - (intptr_t)a);
  // block j of b meets block i of a iff -lb < d + (j - i) s < la
  const int64_t kmin = std::max<int64_t>(floor_div(-lb - d, s) + 1, -(n - 1));
  const int64_t kmax = std::min<int64_t>(floor_div(la - d - 1, s), n - 1);
  return kmin <= kmax;
}

ptdit_status check_common(int64_t B, int64_t D, int64_t heads) {
  if (B < 0 || B > 65535 || D <= 0 || heads <= 0 || heads > 65535) return PTDIT_ERR_SHAPE;
  if (D % heads != 0) return PTDIT_ERR_SHAPE;
  const int64_t dh = D / heads;
  if (dh != 72 && dh != 64) return PTDIT_ERR_SHAPE;  // head widths with compiled kernels
  return PTDIT_OK;
}

ptdit_status check_io_dtypes(ptdit_dtype prec, ptdit_dtype in_dt, ptdit_dtype out_dt) {
  if (!valid_dtype(prec) || !valid_dtype(in_dt) || !valid_dtype(out_dt)) return PTDIT_ERR_DTYPE;
  if (prec == PTDIT_F32 && (in_dt != PTDIT_F32 || out_dt != PTDIT_F32)) return PTDIT_ERR_DTYPE;
  return PTDIT_OK;
}

ptdit_status check_weights(const ptdit_attn_w* w) {
  if (!w || !w->w_qkv || !w->w_o) return PTDIT_ERR_NULL;
  if (!aligned16(w->w_qkv) || !aligned16(w->w_o) || !aligned16(w->b_qkv) || !aligned16(w->b_o) ||
      !aligned16(w->w_qkv_packed))
    return PTDIT_ERR_ALIGN;
  return PTDIT_OK;
}

// Optional bf16 copies of fp32 activations (out_lowp written, x_lowp read):
// only with bf16 precision and an fp32 tensor beside them.
ptdit_status check_lowp(ptdit_dtype prec, const void* lowp, ptdit_dtype beside_dt) {
  if (!lowp) return PTDIT_OK;
  if (prec != PTDIT_BF16 || beside_dt != PTDIT_F32) return PTDIT_ERR_DTYPE;
  return aligned16(lowp) ? PTDIT_OK : PTDIT_ERR_ALIGN;
}

ptdit_status check_grid(const ptdit_grid& g) {
  if (g.F < 0 || g.H < 0 || g.W < 0) return PTDIT_ERR_SHAPE;
  const int64_t N = (int64_t)g.F * g.H * g.W;
  if (N > (int64_t)1 << 30) return PTDIT_ERR_SHAPE;
  return check_common(g.B, g.D, g.heads);
}

hipError_t gemm(ptdit_dtype prec, const void* A, ptdit_dtype a_dt, int64_t M, int K, int N,
                const void* W, const void* bias, const void* R, ptdit_dtype r_dt,
                void* Y, ptdit_dtype y_dt, bool head_major, int64_t Ntok, int heads, int D,
                int trace_cls, hipStream_t s, void* Y2 = nullptr, int act = 0) {
  GemmDesc d;
  d.A = A; d.a_f32 = a_dt == PTDIT_F32;
  d.W = W; d.bias = bias;
  d.R = R; d.r_f32 = r_dt == PTDIT_F32;
  d.Y = Y; d.y_f32 = y_dt == PTDIT_F32;
  d.Y2 = Y2;
  d.M = M; d.N = N; d.K = K;
  d.head_major = head_major; d.Ntok = Ntok; d.heads = heads;
  d.dh = heads > 0 ? D / heads : 0; d.D = D;
  d.act = act;
  TraceScope ts(trace_cls, s);
  return prec == PTDIT_F32 ? launch_gemm_f32(d, s) : launch_gemm_bf16(d, s);
}

const void* offset_elems(const void* p, int64_t elems, ptdit_dtype dt) {
  return p ? (const char*)p + elems * (int64_t)esize(dt) : nullptr;
}

// Window / shifted-window attention shared by both ABI calls.
ptdit_status window_common(const void* x, const void* x_lowp, ptdit_dtype x_dt, ptdit_grid g,
                           ptdit_win3 win, ptdit_win3 shift, const ptdit_attn_w* w,
                           int32_t add_residual, void* out, void* out_lowp, ptdit_dtype out_dt,
                           void* ws, size_t ws_bytes, ptdit_dtype prec, hipStream_t stream, bool keep = false) {
  ptdit_status st = check_grid(g);
  if (st) return st;
  if ((st = check_io_dtypes(prec, x_dt, out_dt))) return st;
  if ((st = check_weights(w))) return st;
  if (win.t <= 0 || win.h <= 0 || win.w <= 0) return PTDIT_ERR_SHAPE;
  if ((int64_t)win.t * win.h * win.w > 128) return PTDIT_ERR_SHAPE;
  if (shift.t < 0 || shift.h < 0 || shift.w < 0 || shift.t >= win.t || shift.h >= win.h ||
      shift.w >= win.w)
    return PTDIT_ERR_SHAPE;
  const int64_t N = (int64_t)g.F * g.H * g.W;
  const int64_t rows = (int64_t)g.B * N;
  if (rows == 0) return PTDIT_OK;
  if (!x || !out) return PTDIT_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws)) return PTDIT_ERR_ALIGN;
  if ((st = check_lowp(prec, x_lowp, x_dt)) || (st = check_lowp(prec, out_lowp, out_dt))) return st;
  const size_t need = ptdit_workspace_bytes(PTDIT_OP_WINDOW_SA, g, 0, win, prec);
  if (!ws || ws_bytes < need) return PTDIT_ERR_WORKSPACE;
  const size_t xb = rows * g.D * esize(x_dt), ob = rows * g.D * esize(out_dt), lb = rows * g.D * 2;
  // inputs must not sit in the workspace either: the Q/K/V projection writes
  // it before the output projection reads x as the residual
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, ws, need) || overlaps(out, ob, x_lowp, lb) ||
      overlaps(out_lowp, lb, x, xb) || overlaps(out_lowp, lb, x_lowp, lb) ||
      overlaps(out_lowp, lb, out, ob) || overlaps(out_lowp, lb, ws, need) || overlaps(x, xb, ws, need) ||
      overlaps(x_lowp, lb, ws, need))
    return PTDIT_ERR_ALIAS;

  const int D = g.D;
  char* wsp = (char*)ws;
  void* qkv = wsp;
  void* o = wsp + align_up((size_t)rows * 3 * D * esize(prec));
  hipError_t e;
  // bf16 operands available as bf16 (x itself, or its copy x_lowp): the
  // Q/K/V projection and the window attention run as one kernel that keeps
  // Q/K/V on chip and writes only the attention output
  const void* xa = x_lowp ? x_lowp : (x_dt == PTDIT_BF16 ? x : nullptr);
  WFusedDesc fd;
  fd.X = xa; fd.w_qkv = w->w_qkv; fd.b_qkv = w->b_qkv; fd.O = o;
  fd.qkv_out = keep ? qkv : nullptr;  // the unfused path writes Q/K/V there anyway
  // the weights packed in the fused kernel's DMA order, after Q/K/V and O
  fd.w_packed = (char*)o + align_up((size_t)rows * D * esize(prec));
  fd.B = g.B; fd.F = g.F; fd.H = g.H; fd.W = g.W; fd.D = D; fd.heads = g.heads; fd.dh = D / g.heads;
  fd.wt = win.t; fd.wh = win.h; fd.ww = win.w;
  fd.st = shift.t; fd.sh = shift.h; fd.sw = shift.w;
  fd.Fp = (g.F + win.t - 1) / win.t * win.t;
  fd.Hp = (g.H + win.h - 1) / win.h * win.h;
  fd.Wp = (g.W + win.w - 1) / win.w * win.w;
  fd.scale = 1.0f / std::sqrt((float)fd.dh);
  if (prec == PTDIT_BF16 && xa && wfused_supported(fd)) {
    if (w->w_qkv_packed) {
      fd.w_packed = const_cast<void*>(w->w_qkv_packed);  // read only
    } else {
      e = launch_wfused_pack(fd, stream);
      if (e != hipSuccess) return PTDIT_ERR_HIP;
    }
    {
      TraceScope ts(PTDIT_K_WINDOW_FUSED, stream);
      e = launch_wfused(fd, stream);
    }
    if (e != hipSuccess) return PTDIT_ERR_HIP;
    e = gemm(prec, o, prec, rows, D, D, w->w_o, w->b_o, add_residual ? x : nullptr, x_dt, out, out_dt,
             false, N, g.heads, D, PTDIT_K_GEMM_OUT, stream, out_lowp);
    return hip_status(e);
  }
  // the projection reads bf16(x); x_lowp, when given, already holds it
  e = gemm(prec, x_lowp ? x_lowp : x, x_lowp ? PTDIT_BF16 : x_dt, rows, D, 3 * D, w->w_qkv,
           w->b_qkv, nullptr, prec, qkv, prec, true, N, g.heads, D, PTDIT_K_GEMM_QKV, stream);
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  WindowDesc wd;
  wd.QKV = qkv; wd.bias_qkv = w->b_qkv; wd.O = o;
  wd.B = g.B; wd.F = g.F; wd.H = g.H; wd.W = g.W; wd.D = D; wd.heads = g.heads; wd.dh = D / g.heads;
  wd.wt = win.t; wd.wh = win.h; wd.ww = win.w;
  wd.st = shift.t; wd.sh = shift.h; wd.sw = shift.w;
  wd.Fp = (g.F + win.t - 1) / win.t * win.t;
  wd.Hp = (g.H + win.h - 1) / win.h * win.h;
  wd.Wp = (g.W + win.w - 1) / win.w * win.w;
  wd.scale = 1.0f / std::sqrt((float)wd.dh);
  {
    TraceScope ts(PTDIT_K_ATTN_WINDOW, stream);
    e = launch_window(wd, prec == PTDIT_F32, stream);
  }
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  e = gemm(prec, o, prec, rows, D, D, w->w_o, w->b_o, add_residual ? x : nullptr, x_dt, out, out_dt,
           false, N, g.heads, D, PTDIT_K_GEMM_OUT, stream, out_lowp);
  return hip_status(e);
}

}  // namespace

extern "C" {

const char* ptdit_version(void) { return "ptdit-mi355x 0.1 (gfx950)"; }

const char* ptdit_status_str(ptdit_status st) {
  switch (st) {
    case PTDIT_OK: return "ok";
    case PTDIT_ERR_NULL: return "null pointer";
    case PTDIT_ERR_SHAPE: return "invalid shape";
    case PTDIT_ERR_DIVISIBILITY: return "proxy window does not divide the grid";
    case PTDIT_ERR_DTYPE: return "unsupported dtype combination";
    case PTDIT_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PTDIT_ERR_WORKSPACE: return "workspace missing or too small";
    case PTDIT_ERR_HIP: return "HIP launch failed";
    case PTDIT_ERR_ALIAS: return "output overlaps an input or the workspace";
    case PTDIT_ERR_SCRATCH: return "problem too large for the static scratch of the no-allocation entry point";
  }
  return "unknown status";
}

size_t ptdit_workspace_bytes(ptdit_op op, ptdit_grid g, int32_t M, ptdit_win3 win, ptdit_dtype prec) {
  if (!valid_dtype(prec) || g.B < 0 || g.D <= 0 || g.F < 0 || g.H < 0 || g.W < 0) return 0;
  const size_t es = esize(prec);
  const size_t B = (size_t)g.B, D = (size_t)g.D;
  const size_t N = (size_t)g.F * g.H * g.W;
  switch (op) {
    case PTDIT_OP_PROXY_SA:
      if (M < 0) return 0;
      return align_up(B * 3 * M * D * es) + align_up(B * M * D * es);
    case PTDIT_OP_PROXY_XATTN:
      if (M < 0) return 0;
      // Q, K/V, attention output, and (bf16, more than 512 keys) packed V^T blocks
      return align_up(B * N * D * es) + align_up(B * 2 * M * D * es) + align_up(B * N * D * es) +
             (prec == PTDIT_BF16 && g.heads > 0 ? align_up(ptdit::flash_vt_bytes(g.B, g.heads, M)) : 0);
    case PTDIT_OP_WINDOW_SA:
    case PTDIT_OP_SHIFT_WINDOW_SA:
      // windows the calls reject need no workspace: 0 (invalid arguments)
      if (win.t <= 0 || win.h <= 0 || win.w <= 0 || (int64_t)win.t * win.h * win.w > 128) return 0;
      // Q/K/V and the attention output (the fused kernel uses only the
      // latter), then (bf16) w_qkv packed for the fused kernel, 3 D^2 bf16
      return align_up(B * 3 * N * D * es) + align_up(B * N * D * es) +
             (prec == PTDIT_BF16 ? align_up(3 * D * D * 2) : 0);
    case PTDIT_OP_MLP:
      if (M <= 0) return 0;
      return align_up(B * N * (size_t)M * es);
  }
  return 0;
}

ptdit_status ptdit_linear(const void* x, ptdit_dtype x_dt, int64_t rows, int32_t d_in,
                          int32_t d_out, const void* w, const void* b,
                          const void* residual, ptdit_dtype r_dt,
                          void* y, ptdit_dtype y_dt, ptdit_dtype prec, hipStream_t stream) {
  if (!valid_dtype(prec) || !valid_dtype(x_dt) || !valid_dtype(y_dt) || !valid_dtype(r_dt))
    return PTDIT_ERR_DTYPE;
  if (prec == PTDIT_F32 && (x_dt != PTDIT_F32 || y_dt != PTDIT_F32 || (residual && r_dt != PTDIT_F32)))
    return PTDIT_ERR_DTYPE;
  if (rows < 0 || d_in <= 0 || d_out <= 0 || d_in % 8 || d_out % 8) return PTDIT_ERR_SHAPE;
  if (rows == 0) return PTDIT_OK;
  if (!x || !w || !y) return PTDIT_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(b) || !aligned16(residual) || !aligned16(y))
    return PTDIT_ERR_ALIGN;
  if (overlaps(y, rows * d_out * esize(y_dt), x, rows * d_in * esize(x_dt))) return PTDIT_ERR_ALIAS;
  hipError_t e = gemm(prec, x, x_dt, rows, d_in, d_out, w, b, residual, r_dt, y, y_dt, false, rows, 1,
                      d_out, PTDIT_K_GEMM_OUT, stream);
  return hip_status(e);
}

ptdit_status ptdit_proxy_pool(const void* x, ptdit_dtype x_dt, ptdit_grid g, ptdit_win3 p,
                              void* proxies, ptdit_dtype out_dt, hipStream_t stream) {
  if (!valid_dtype(x_dt) || !valid_dtype(out_dt)) return PTDIT_ERR_DTYPE;
  if (g.B < 0 || g.F < 0 || g.H < 0 || g.W < 0 || g.D <= 0 || g.D % 8) return PTDIT_ERR_SHAPE;
  if (p.t <= 0 || p.h <= 0 || p.w <= 0) return PTDIT_ERR_SHAPE;
  if (g.F % p.t || g.H % p.h || g.W % p.w) return PTDIT_ERR_DIVISIBILITY;
  const int64_t N = (int64_t)g.F * g.H * g.W;
  if (N > (int64_t)1 << 30) return PTDIT_ERR_SHAPE;
  const int64_t M = N / ((int64_t)p.t * p.h * p.w);
  if ((int64_t)g.B * M > INT32_MAX) return PTDIT_ERR_SHAPE;
  if ((int64_t)g.B * M == 0) return PTDIT_OK;
  if (!x || !proxies) return PTDIT_ERR_NULL;
  if (!aligned16(x) || !aligned16(proxies)) return PTDIT_ERR_ALIGN;
  if (overlaps(proxies, g.B * M * g.D * esize(out_dt), x, g.B * N * g.D * esize(x_dt)))
    return PTDIT_ERR_ALIAS;
  PoolDesc d;
  d.x = x; d.x_f32 = x_dt == PTDIT_F32;
  d.out = proxies; d.out_f32 = out_dt == PTDIT_F32;
  d.B = g.B; d.F = g.F; d.H = g.H; d.W = g.W; d.D = g.D;
  d.pt = p.t; d.ph = p.h; d.pw = p.w;
  TraceScope ts(PTDIT_K_POOL, stream);
  return hip_status(launch_pool(d, stream));
}

ptdit_status ptdit_mlp(const void* x, const void* x_lowp, ptdit_dtype x_dt, int64_t rows, int32_t D,
                       int32_t hidden, const ptdit_mlp_w* w, int32_t add_residual, void* out,
                       void* out_lowp, ptdit_dtype out_dt, void* ws, size_t ws_bytes, ptdit_dtype prec,
                       hipStream_t stream) {
  ptdit_status st = check_io_dtypes(prec, x_dt, out_dt);
  if (st) return st;
  if (rows < 0 || D <= 0 || hidden <= 0 || D % 8 || hidden % 8) return PTDIT_ERR_SHAPE;
  if (!w || !w->w1 || !w->w2) return PTDIT_ERR_NULL;
  if (rows == 0) return PTDIT_OK;
  if (!x || !out) return PTDIT_ERR_NULL;
  if (x_lowp && (prec != PTDIT_BF16 || x_dt != PTDIT_F32)) return PTDIT_ERR_DTYPE;
  if ((st = check_lowp(prec, out_lowp, out_dt))) return st;
  if (!aligned16(x) || !aligned16(x_lowp) || !aligned16(out) || !aligned16(ws) || !aligned16(w->w1) ||
      !aligned16(w->w2) || !aligned16(w->b1) || !aligned16(w->b2))
    return PTDIT_ERR_ALIGN;
  const ptdit_grid g{(int32_t)std::min<int64_t>(rows, INT32_MAX), 1, 1, 1, D, 1};
  if (rows > INT32_MAX) return PTDIT_ERR_SHAPE;
  const size_t need = ptdit_workspace_bytes(PTDIT_OP_MLP, g, hidden, ptdit_win3{1, 1, 1}, prec);
  if (!ws || ws_bytes < need) return PTDIT_ERR_WORKSPACE;
  const size_t xb = rows * D * esize(x_dt), ob = rows * D * esize(out_dt), lb = rows * D * 2;
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, ws, need) || overlaps(out, ob, x_lowp, lb) ||
      overlaps(out_lowp, lb, x, xb) || overlaps(out_lowp, lb, x_lowp, lb) || overlaps(out_lowp, lb, out, ob) ||
      overlaps(out_lowp, lb, ws, need) || overlaps(x, xb, ws, need) || overlaps(x_lowp, lb, ws, need))
    return PTDIT_ERR_ALIAS;
  // h = GELU(x W1^T + b1) into the workspace, then out = h W2^T + b2 (+ x)
  hipError_t e = gemm(prec, x_lowp ? x_lowp : x, x_lowp ? PTDIT_BF16 : x_dt, rows, D, hidden, w->w1, w->b1,
                      nullptr, prec, ws, prec, false, rows, 1, hidden, PTDIT_K_GEMM_MLP, stream, nullptr, 1);
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  e = gemm(prec, ws, prec, rows, hidden, D, w->w2, w->b2, add_residual ? x : nullptr, x_dt, out, out_dt, false,
           rows, 1, D, PTDIT_K_GEMM_MLP, stream, out_lowp);
  return hip_status(e);
}

ptdit_status ptdit_proxy_select(const void* x, ptdit_dtype x_dt, ptdit_grid g, ptdit_win3 p,
                                const int32_t* offsets, void* proxies, ptdit_dtype out_dt,
                                hipStream_t stream) {
  if (!valid_dtype(x_dt) || !valid_dtype(out_dt)) return PTDIT_ERR_DTYPE;
  if (g.B < 0 || g.F < 0 || g.H < 0 || g.W < 0 || g.D <= 0 || g.D % 8) return PTDIT_ERR_SHAPE;
  if (p.t <= 0 || p.h <= 0 || p.w <= 0) return PTDIT_ERR_SHAPE;
  if (g.F % p.t || g.H % p.h || g.W % p.w) return PTDIT_ERR_DIVISIBILITY;
  const int64_t N = (int64_t)g.F * g.H * g.W;
  if (N > (int64_t)1 << 30) return PTDIT_ERR_SHAPE;
  const int64_t M = N / ((int64_t)p.t * p.h * p.w);
  if ((int64_t)g.B * M > INT32_MAX) return PTDIT_ERR_SHAPE;
  if ((int64_t)g.B * M == 0) return PTDIT_OK;
  if (!x || !proxies) return PTDIT_ERR_NULL;
  if (!aligned16(x) || !aligned16(proxies) || ((uintptr_t)offsets & 3)) return PTDIT_ERR_ALIGN;
  const size_t pb = g.B * M * g.D * esize(out_dt);
  if (overlaps(proxies, pb, x, g.B * N * g.D * esize(x_dt)) ||
      overlaps(proxies, pb, offsets, (size_t)g.B * M * sizeof(int32_t)))
    return PTDIT_ERR_ALIAS;
  PoolDesc d;
  d.x = x; d.x_f32 = x_dt == PTDIT_F32;
  d.out = proxies; d.out_f32 = out_dt == PTDIT_F32;
  d.B = g.B; d.F = g.F; d.H = g.H; d.W = g.W; d.D = g.D;
  d.pt = p.t; d.ph = p.h; d.pw = p.w;
  TraceScope ts(PTDIT_K_POOL, stream);
  return hip_status(launch_select(d, offsets, stream));
}

ptdit_status ptdit_proxy_sa(const void* proxies, ptdit_dtype p_dt, int32_t B, int32_t M,
                            int32_t D, int32_t heads, const ptdit_attn_w* w,
                            int32_t add_residual, void* out, ptdit_dtype out_dt,
                            void* ws, size_t ws_bytes, ptdit_dtype prec, hipStream_t stream) {
  ptdit_status st = check_common(B, D, heads);
  if (st) return st;
  if (M < 0) return PTDIT_ERR_SHAPE;
  if ((st = check_io_dtypes(prec, p_dt, out_dt))) return st;
  if ((st = check_weights(w))) return st;
  const int64_t rows = (int64_t)B * M;
  if (rows == 0) return PTDIT_OK;
  if (!proxies || !out) return PTDIT_ERR_NULL;
  if (!aligned16(proxies) || !aligned16(out) || !aligned16(ws)) return PTDIT_ERR_ALIGN;
  ptdit_grid g{B, 1, 1, M, D, heads};
  const size_t need = ptdit_workspace_bytes(PTDIT_OP_PROXY_SA, g, M, ptdit_win3{1, 1, 1}, prec);
  if (!ws || ws_bytes < need) return PTDIT_ERR_WORKSPACE;
  if (overlaps(out, rows * D * esize(out_dt), proxies, rows * D * esize(p_dt)) ||
      overlaps(out, rows * D * esize(out_dt), ws, need) || overlaps(proxies, rows * D * esize(p_dt), ws, need))
    return PTDIT_ERR_ALIAS;

  const int dh = D / heads;
  char* wsp = (char*)ws;
  void* qkv = wsp;
  void* o = wsp + align_up((size_t)rows * 3 * D * esize(prec));
  hipError_t e = gemm(prec, proxies, p_dt, rows, D, 3 * D, w->w_qkv, w->b_qkv, nullptr, prec, qkv,
                      prec, true, M, heads, D, PTDIT_K_GEMM_PROXY, stream);
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  FlashDesc f;
  const int64_t hs = (int64_t)M * dh, gs = (int64_t)heads * hs;
  f.Q = qkv; f.q_bs = 3 * gs; f.q_hs = hs;
  f.K = offset_elems(qkv, gs, prec); f.k_bs = 3 * gs; f.k_hs = hs;
  f.V = offset_elems(qkv, 2 * gs, prec); f.v_bs = 3 * gs; f.v_hs = hs;
  f.O = o; f.B = B; f.heads = heads; f.Nq = M; f.Nk = M; f.dh = dh; f.D = D;
  f.scale = 1.0f / std::sqrt((float)dh);
  {
    TraceScope ts(PTDIT_K_ATTN_FLASH, stream);
    e = launch_flash(f, prec == PTDIT_F32, stream);
  }
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  e = gemm(prec, o, prec, rows, D, D, w->w_o, w->b_o, add_residual ? proxies : nullptr, p_dt, out,
           out_dt, false, M, heads, D, PTDIT_K_GEMM_PROXY, stream);
  return hip_status(e);
}

// ------------------------------------------------------------------ no-allocation proxy SA
// Scratch of ptdit_proxy_sa_noalloc: the Q/K/V and attention-output
// workspace of ptdit_proxy_sa, in a file-scope device array that every GPU
// the library runs on holds until the process ends. Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in
// for the symbol): it uses the device address hipGetSymbolAddress returns,
// looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[PTDIT_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of this device's scratch (nullptr on failure)
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

ptdit_status ptdit_proxy_sa_noalloc(const void* proxies, ptdit_dtype p_dt, int32_t B, int32_t M,
                                    int32_t D, int32_t heads, const ptdit_attn_w* w,
                                    int32_t add_residual, void* out, ptdit_dtype out_dt,
                                    ptdit_dtype prec, hipStream_t stream) {
  ptdit_status st = check_common(B, D, heads);
  if (st) return st;
  if (M < 0) return PTDIT_ERR_SHAPE;
  if (!valid_dtype(prec)) return PTDIT_ERR_DTYPE;
  if ((int64_t)B * M == 0) return PTDIT_OK;
  const ptdit_grid g{B, 1, 1, M, D, heads};
  const size_t need = ptdit_workspace_bytes(PTDIT_OP_PROXY_SA, g, M, ptdit_win3{1, 1, 1}, prec);
  if (need == 0 || need > (size_t)PTDIT_NOALLOC_SCRATCH_BYTES) return PTDIT_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PTDIT_ERR_HIP;
  void* ws = scratch_address(dev);
  if (!ws) return PTDIT_ERR_HIP;
  // the same kernels as ptdit_proxy_sa: the projection writes every Q/K/V
  // element and the attention core every output element before they are
  // read, so nothing of a previous call's scratch contents is used
  return ptdit_proxy_sa(proxies, p_dt, B, M, D, heads, w, add_residual, out, out_dt, ws,
                        (size_t)PTDIT_NOALLOC_SCRATCH_BYTES, prec, stream);
}

ptdit_status ptdit_proxy_xattn(const void* x, const void* x_lowp, ptdit_dtype x_dt, ptdit_grid g,
                               const void* proxies, ptdit_dtype p_dt, int32_t M,
                               const ptdit_attn_w* w, int32_t add_residual,
                               void* out, void* out_lowp, ptdit_dtype out_dt,
                               void* ws, size_t ws_bytes, ptdit_dtype prec, hipStream_t stream) {
  ptdit_status st = check_grid(g);
  if (st) return st;
  if ((st = check_io_dtypes(prec, x_dt, out_dt))) return st;
  if (!valid_dtype(p_dt) || (prec == PTDIT_F32 && p_dt != PTDIT_F32)) return PTDIT_ERR_DTYPE;
  if ((st = check_weights(w))) return st;
  const int64_t N = (int64_t)g.F * g.H * g.W;
  const int64_t rows = (int64_t)g.B * N;
  if (rows == 0) return PTDIT_OK;
  if (M <= 0) return PTDIT_ERR_SHAPE;  // softmax over an empty key set is undefined
  if (!x || !proxies || !out) return PTDIT_ERR_NULL;
  if (!aligned16(x) || !aligned16(proxies) || !aligned16(out) || !aligned16(ws)) return PTDIT_ERR_ALIGN;
  if ((st = check_lowp(prec, out_lowp, out_dt))) return st;
  if ((st = check_lowp(prec, x_lowp, x_dt))) return st;
  const size_t need = ptdit_workspace_bytes(PTDIT_OP_PROXY_XATTN, g, M, ptdit_win3{1, 1, 1}, prec);
  if (!ws || ws_bytes < need) return PTDIT_ERR_WORKSPACE;
  const size_t ob = rows * g.D * esize(out_dt), lb = rows * g.D * 2;
  const size_t xb = rows * g.D * esize(x_dt), pb = (size_t)g.B * M * g.D * esize(p_dt);
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, proxies, pb) || overlaps(out, ob, ws, need) ||
      overlaps(out_lowp, lb, x, xb) || overlaps(out_lowp, lb, proxies, pb) ||
      overlaps(out_lowp, lb, out, ob) || overlaps(out_lowp, lb, ws, need) || overlaps(out, ob, x_lowp, lb) ||
      overlaps(out_lowp, lb, x_lowp, lb) || overlaps(x, xb, ws, need) || overlaps(x_lowp, lb, ws, need) ||
      overlaps(proxies, pb, ws, need))
    return PTDIT_ERR_ALIAS;

  const int D = g.D, heads = g.heads, dh = D / heads;
  const size_t es = esize(prec);
  char* wsp = (char*)ws;
  void* q = wsp;
  void* kv = wsp + align_up((size_t)rows * D * es);
  void* o = (char*)kv + align_up((size_t)g.B * 2 * M * D * es);
  // Q = x Wq^T + bq (rows 0..D-1 of w_qkv), head-major [B][1][heads][N][dh];
  // the projection reads bf16(x), which x_lowp, when given, already holds
  hipError_t e = gemm(prec, x_lowp ? x_lowp : x, x_lowp ? PTDIT_BF16 : x_dt, rows, D, D, w->w_qkv, w->b_qkv,
                      nullptr, prec, q, prec, true, N, heads, D, PTDIT_K_GEMM_Q, stream);
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  // K, V = P' W_{k,v}^T + b_{k,v} (rows D..3D-1), head-major [B][2][heads][M][dh]
  e = gemm(prec, proxies, p_dt, (int64_t)g.B * M, D, 2 * D, offset_elems(w->w_qkv, (int64_t)D * D, prec),
           offset_elems(w->b_qkv, D, prec), nullptr, prec, kv, prec, true, M, heads, D,
           PTDIT_K_GEMM_PROXY, stream);
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  FlashDesc f;
  const int64_t qhs = N * dh, khs = (int64_t)M * dh;
  f.Q = q; f.q_bs = heads * qhs; f.q_hs = qhs;
  f.K = kv; f.k_bs = 2 * heads * khs; f.k_hs = khs;
  f.V = offset_elems(kv, heads * khs, prec); f.v_bs = 2 * heads * khs; f.v_hs = khs;
  f.O = o; f.B = g.B; f.heads = heads; f.Nq = (int)N; f.Nk = M; f.dh = dh; f.D = D;
  f.scale = 1.0f / std::sqrt((float)dh);
  if (prec == PTDIT_BF16) {
    f.vt = (char*)o + align_up((size_t)rows * D * es);
    f.vt_bytes = flash_vt_bytes(g.B, heads, M);
  }
  {
    TraceScope ts(PTDIT_K_ATTN_FLASH, stream);
    e = launch_flash(f, prec == PTDIT_F32, stream);
  }
  if (e != hipSuccess) return PTDIT_ERR_HIP;
  e = gemm(prec, o, prec, rows, D, D, w->w_o, w->b_o, add_residual ? x : nullptr, x_dt, out, out_dt,
           false, N, heads, D, PTDIT_K_GEMM_OUT, stream, out_lowp);
  return hip_status(e);
}

// the fused kernel's weight layout for (D, heads): the descriptor fields the
// packing and wfused_supported read (one 64-token window, one token)
static WFusedDesc pack_desc(int32_t D, int32_t heads) {
  WFusedDesc fd{};
  fd.B = 1; fd.F = 1; fd.H = 8; fd.W = 8; fd.D = D; fd.heads = heads; fd.dh = heads > 0 ? D / heads : 0;
  fd.wt = 1; fd.wh = 8; fd.ww = 8;
  fd.Fp = 1; fd.Hp = 8; fd.Wp = 8;
  return fd;
}

size_t ptdit_window_packed_bytes(int32_t D, int32_t heads) {
  if (D <= 0 || heads <= 0 || D % heads) return 0;
  return wfused_supported(pack_desc(D, heads)) ? wfused_packed_bytes(D) : 0;
}

ptdit_status ptdit_pack_window_weights(const void* w_qkv, int32_t D, int32_t heads, void* packed,
                                       hipStream_t stream) {
  if (!w_qkv || !packed) return PTDIT_ERR_NULL;
  if (!aligned16(w_qkv) || !aligned16(packed)) return PTDIT_ERR_ALIGN;
  const size_t nb = ptdit_window_packed_bytes(D, heads);
  if (nb == 0) return PTDIT_ERR_SHAPE;
  if (overlaps(packed, nb, w_qkv, (size_t)3 * D * D * 2)) return PTDIT_ERR_ALIAS;
  WFusedDesc fd = pack_desc(D, heads);
  fd.w_qkv = w_qkv;
  fd.w_packed = packed;
  return hip_status(launch_wfused_pack(fd, stream));
}

ptdit_status ptdit_window_sa(const void* x, const void* x_lowp, ptdit_dtype x_dt, ptdit_grid g,
                             ptdit_win3 win, const ptdit_attn_w* w, int32_t add_residual,
                             void* out, void* out_lowp, ptdit_dtype out_dt,
                             void* ws, size_t ws_bytes, ptdit_dtype prec, hipStream_t stream) {
  return window_common(x, x_lowp, x_dt, g, win, ptdit_win3{0, 0, 0}, w, add_residual, out, out_lowp,
                       out_dt, ws, ws_bytes, prec, stream);
}

ptdit_status ptdit_shift_window_sa(const void* x, const void* x_lowp, ptdit_dtype x_dt,
                                   ptdit_grid g, ptdit_win3 win, ptdit_win3 shift,
                                   const ptdit_attn_w* w, int32_t add_residual,
                                   void* out, void* out_lowp, ptdit_dtype out_dt,
                                   void* ws, size_t ws_bytes, ptdit_dtype prec,
                                   hipStream_t stream) {
  return window_common(x, x_lowp, x_dt, g, win, shift, w, add_residual, out, out_lowp, out_dt, ws,
                       ws_bytes, prec, stream);
}

ptdit_status ptdit_window_sa_keep(const void* x, const void* x_lowp, ptdit_dtype x_dt, ptdit_grid g,
                                  ptdit_win3 win, ptdit_win3 shift, const ptdit_attn_w* w, int32_t add_residual,
                                  void* out, void* out_lowp, ptdit_dtype out_dt, void* ws, size_t ws_bytes,
                                  ptdit_dtype prec, hipStream_t stream) {
  return window_common(x, x_lowp, x_dt, g, win, shift, w, add_residual, out, out_lowp, out_dt, ws, ws_bytes, prec,
                       stream, true);
}

ptdit_status ptdit_roll3d(const void* x, ptdit_grid g, ptdit_win3 shift, int32_t inverse,
                          void* y, ptdit_dtype dt, hipStream_t stream) {
  if (!valid_dtype(dt)) return PTDIT_ERR_DTYPE;
  if (g.B < 0 || g.F < 0 || g.H < 0 || g.W < 0 || g.D <= 0 || g.D % 8) return PTDIT_ERR_SHAPE;
  if (shift.t < 0 || shift.h < 0 || shift.w < 0) return PTDIT_ERR_SHAPE;
  const int64_t N = (int64_t)g.F * g.H * g.W;
  if (N > (int64_t)1 << 30) return PTDIT_ERR_SHAPE;
  if (g.B * N == 0) return PTDIT_OK;
  // the kernel indexes grid rows (b, t, i) and the 16-byte vectors of one row in 32 bits
  const int64_t vec_per_row = (int64_t)g.W * g.D * esize(dt) / 16;
  if ((int64_t)g.B * g.F * g.H > INT32_MAX || vec_per_row > INT32_MAX - 1024) return PTDIT_ERR_SHAPE;
  if (!x || !y) return PTDIT_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return PTDIT_ERR_ALIGN;
  const size_t bytes = g.B * N * g.D * esize(dt);
  if (overlaps(x, bytes, y, bytes)) return PTDIT_ERR_ALIAS;
  auto norm = [&](int s, int L) {
    int r = s % L;
    if (inverse) r = (L - r) % L;
    return r;
  };
  RollDesc d;
  d.x = x; d.y = y; d.f32 = dt == PTDIT_F32;
  d.B = g.B; d.F = g.F; d.H = g.H; d.W = g.W; d.D = g.D;
  d.st = norm(shift.t, g.F); d.sh = norm(shift.h, g.H); d.sw = norm(shift.w, g.W);
  TraceScope ts(PTDIT_K_ROLL, stream);
  return hip_status(launch_roll(d, stream));
}

static ptdit_status window_attn_bwd(const void* qkv, const void* b_qkv, const void* d_o, ptdit_dtype dt,
                                    ptdit_grid g, ptdit_win3 win, ptdit_win3 shift, void* d_qkv,
                                    ptdit_dtype out_dt, float* d_b_kv, int tokens_out, hipStream_t stream) {
  if (!valid_dtype(dt) || !valid_dtype(out_dt)) return PTDIT_ERR_DTYPE;
  if (out_dt == PTDIT_BF16 && dt != PTDIT_BF16) return PTDIT_ERR_DTYPE;  // bf16 gradients from bf16 inputs
  ptdit_status st = check_grid(g);
  if (st) return st;
  if (win.t <= 0 || win.h <= 0 || win.w <= 0) return PTDIT_ERR_SHAPE;
  if ((int64_t)win.t * win.h * win.w > 128) return PTDIT_ERR_SHAPE;
  if (shift.t < 0 || shift.h < 0 || shift.w < 0 || shift.t >= win.t || shift.h >= win.h ||
      shift.w >= win.w)
    return PTDIT_ERR_SHAPE;
  const int64_t N = (int64_t)g.F * g.H * g.W, rows = (int64_t)g.B * N;
  if (rows == 0) return PTDIT_OK;
  const bool pads = g.F % win.t || g.H % win.h || g.W % win.w;
  if (!qkv || !d_o || !d_qkv || (pads && !d_b_kv)) return PTDIT_ERR_NULL;
  if (!aligned16(qkv) || !aligned16(d_o) || !aligned16(d_qkv) || !aligned16(b_qkv) || !aligned16(d_b_kv))
    return PTDIT_ERR_ALIGN;
  const size_t gb = (size_t)rows * 3 * g.D * esize(out_dt), bb = (size_t)2 * g.D * 4;
  if (overlaps(d_qkv, gb, qkv, rows * 3 * g.D * esize(dt)) || overlaps(d_qkv, gb, d_o, rows * g.D * esize(dt)) ||
      overlaps(d_qkv, gb, b_qkv, 3 * g.D * esize(dt)) || overlaps(d_b_kv, bb, d_qkv, gb) ||
      overlaps(d_b_kv, bb, qkv, rows * 3 * g.D * esize(dt)) || overlaps(d_b_kv, bb, d_o, rows * g.D * esize(dt)))
    return PTDIT_ERR_ALIAS;
  WindowBwdDesc d;
  d.QKV = qkv; d.bias_qkv = b_qkv; d.dO = d_o; d.dQKV = d_qkv; d.dbias_kv = d_b_kv;
  d.tokens_out = tokens_out;
  d.out_bf16 = out_dt == PTDIT_BF16;
  d.B = g.B; d.F = g.F; d.H = g.H; d.W = g.W; d.D = g.D; d.heads = g.heads; d.dh = g.D / g.heads;
  d.wt = win.t; d.wh = win.h; d.ww = win.w;
  d.st = shift.t; d.sh = shift.h; d.sw = shift.w;
  d.Fp = (g.F + win.t - 1) / win.t * win.t;
  d.Hp = (g.H + win.h - 1) / win.h * win.h;
  d.Wp = (g.W + win.w - 1) / win.w * win.w;
  d.scale = 1.0f / std::sqrt((float)d.dh);
  TraceScope ts(PTDIT_K_BWD_WINDOW, stream);
  return hip_status(launch_window_bwd(d, dt == PTDIT_F32, stream));
}

ptdit_status ptdit_window_attn_bwd(const void* qkv, const void* b_qkv, const void* d_o, ptdit_dtype dt,
                                   ptdit_grid g, ptdit_win3 win, ptdit_win3 shift, float* d_qkv,
                                   float* d_b_kv, hipStream_t stream) {
  return window_attn_bwd(qkv, b_qkv, d_o, dt, g, win, shift, d_qkv, PTDIT_F32, d_b_kv, 0, stream);
}

ptdit_status ptdit_window_attn_bwd_tokens(const void* qkv, const void* b_qkv, const void* d_o, ptdit_dtype dt,
                                          ptdit_grid g, ptdit_win3 win, ptdit_win3 shift, void* d_qkv_t,
                                          ptdit_dtype d_qkv_dt, float* d_b_kv, hipStream_t stream) {
  return window_attn_bwd(qkv, b_qkv, d_o, dt, g, win, shift, d_qkv_t, d_qkv_dt, d_b_kv, 1, stream);
}

namespace {
constexpr int kBwdQChunk = 1024;  // queries per partial-sum chunk of the key-major kernel
int bwd_chunks(int Nq) { return Nq <= kBwdQChunk ? 1 : (Nq + kBwdQChunk - 1) / kBwdQChunk; }
}  // namespace

size_t ptdit_attn_bwd_workspace_bytes(int32_t B, int32_t heads, int32_t Nq, int32_t Nk, int32_t dh) {
  if (B < 0 || heads <= 0 || Nq < 0 || Nk < 0 || (dh != 64 && dh != 72)) return 0;
  const int chunks = bwd_chunks(Nq);
  size_t bytes = align_up((size_t)B * heads * Nq * 3 * 4);
  if (chunks > 1) bytes += align_up((size_t)chunks * B * heads * Nk * 2 * dh * 4);
  return bytes < kAlign ? kAlign : bytes;
}

static ptdit_status attn_bwd(const void* q, int64_t q_bstride, const void* k, const void* v,
                             int64_t kv_bstride, const void* d_o, ptdit_dtype dt, int32_t B, int32_t heads,
                             int32_t Nq, int32_t Nk, int32_t dh, void* d_q, int64_t dq_bstride, int dq_tok,
                             ptdit_dtype dq_dt, float* d_k, float* d_v, int64_t dkv_bstride, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dt) || !valid_dtype(dq_dt)) return PTDIT_ERR_DTYPE;
  if (dq_dt == PTDIT_BF16 && dt != PTDIT_BF16) return PTDIT_ERR_DTYPE;  // bf16 gradients from bf16 inputs
  if (B < 0 || heads <= 0 || Nq < 0 || Nk < 0 || (dh != 64 && dh != 72)) return PTDIT_ERR_SHAPE;
  if ((int64_t)B * heads > 65535 || Nq > (1 << 30) || (Nq > 0 && Nk == 0) || bwd_chunks(Nq) > 65535)
    return PTDIT_ERR_SHAPE;
  if ((int64_t)B * Nq == 0) return PTDIT_OK;
  const int64_t hq = (int64_t)heads * Nq * dh, hk = (int64_t)heads * Nk * dh;
  if (q_bstride < hq || kv_bstride < hk || dq_bstride < hq || dkv_bstride < hk) return PTDIT_ERR_SHAPE;
  if (!q || !k || !v || !d_o || !d_q || !d_k || !d_v) return PTDIT_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(d_q) ||
      !aligned16(d_k) || !aligned16(d_v) || !aligned16(ws))
    return PTDIT_ERR_ALIGN;
  const size_t need = ptdit_attn_bwd_workspace_bytes(B, heads, Nq, Nk, dh);
  if (!ws || ws_bytes < need) return PTDIT_ERR_WORKSPACE;
  // every operand as B batch blocks (stride, bytes); d_o and ws are one block
  const int64_t es = (int64_t)esize(dt);
  struct Blk { const void* p; int64_t stride, len, n; };
  const Blk ins[4] = {{q, q_bstride * es, hq * es, B}, {k, kv_bstride * es, hk * es, B},
                      {v, kv_bstride * es, hk * es, B}, {d_o, 0, (int64_t)B * Nq * heads * dh * es, 1}};
  const int64_t qes = (int64_t)esize(dq_dt);
  const Blk outs[4] = {{d_q, dq_bstride * qes, hq * qes, B}, {d_k, dkv_bstride * 4, hk * 4, B},
                       {d_v, dkv_bstride * 4, hk * 4, B}, {ws, 0, (int64_t)need, 1}};
  auto meet = [](const Blk& x, const Blk& y) {
    if (x.n == y.n) return overlaps_strided(x.p, x.stride, x.len, y.p, y.stride, y.len, x.n);
    return overlaps(x.p, (size_t)((x.n - 1) * x.stride + x.len), y.p, (size_t)((y.n - 1) * y.stride + y.len));
  };
  for (int a = 0; a < 4; ++a) {
    for (int c = 0; c < 4; ++c)
      if (meet(outs[a], ins[c])) return PTDIT_ERR_ALIAS;
    for (int c = a + 1; c < 4; ++c)
      if (meet(outs[a], outs[c])) return PTDIT_ERR_ALIAS;
  }
  DenseBwdDesc d;
  d.q = q; d.k = k; d.v = v; d.dO = d_o;
  d.q_bs = q_bstride; d.kv_bs = kv_bstride;
  d.dq = d_q; d.dk = d_k; d.dv = d_v; d.dq_bs = dq_bstride; d.dkv_bs = dkv_bstride;
  d.dq_tok = dq_tok; d.dq_bf16 = dq_dt == PTDIT_BF16;
  d.stats = (float*)ws;
  d.part = (float*)((char*)ws + align_up((size_t)B * heads * Nq * 3 * 4));
  d.B = B; d.heads = heads; d.Nq = Nq; d.Nk = Nk; d.D = heads * dh; d.dh = dh;
  d.chunks = bwd_chunks(Nq);
  d.qchunk = d.chunks == 1 ? Nq : kBwdQChunk;
  d.scale = 1.0f / std::sqrt((float)dh);
  TraceScope ts(PTDIT_K_BWD_DENSE, stream);
  return hip_status(launch_dense_bwd(d, dt == PTDIT_F32, stream));
}

ptdit_status ptdit_attn_bwd(const void* q, int64_t q_bstride, const void* k, const void* v,
                            int64_t kv_bstride, const void* d_o, ptdit_dtype dt, int32_t B, int32_t heads,
                            int32_t Nq, int32_t Nk, int32_t dh, float* d_q, int64_t dq_bstride, float* d_k,
                            float* d_v, int64_t dkv_bstride, void* ws, size_t ws_bytes, hipStream_t stream) {
  return attn_bwd(q, q_bstride, k, v, kv_bstride, d_o, dt, B, heads, Nq, Nk, dh, d_q, dq_bstride, 0, PTDIT_F32,
                  d_k, d_v, dkv_bstride, ws, ws_bytes, stream);
}

ptdit_status ptdit_attn_bwd_tokens(const void* q, int64_t q_bstride, const void* k, const void* v,
                                   int64_t kv_bstride, const void* d_o, ptdit_dtype dt, int32_t B, int32_t heads,
                                   int32_t Nq, int32_t Nk, int32_t dh, void* d_q_t, ptdit_dtype d_q_dt, float* d_k,
                                   float* d_v, int64_t dkv_bstride, void* ws, size_t ws_bytes, hipStream_t stream) {
  return attn_bwd(q, q_bstride, k, v, kv_bstride, d_o, dt, B, heads, Nq, Nk, dh, d_q_t,
                  (int64_t)Nq * heads * dh, 1, d_q_dt, d_k, d_v, dkv_bstride, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ recompute and chaining calls
ptdit_status ptdit_linear_heads(const void* x, ptdit_dtype x_dt, int32_t B, int32_t Ntok, int32_t D,
                                int32_t groups, int32_t heads, const void* w, const void* b, void* y,
                                ptdit_dtype prec, hipStream_t stream) {
  if (!valid_dtype(prec) || !valid_dtype(x_dt)) return PTDIT_ERR_DTYPE;
  if (prec == PTDIT_F32 && x_dt != PTDIT_F32) return PTDIT_ERR_DTYPE;
  ptdit_status st = check_common(B, D, heads);
  if (st) return st;
  if (Ntok < 0 || groups < 1 || groups > 3) return PTDIT_ERR_SHAPE;
  const int64_t rows = (int64_t)B * Ntok;
  if (rows == 0) return PTDIT_OK;
  if (!x || !w || !y) return PTDIT_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(b) || !aligned16(y)) return PTDIT_ERR_ALIGN;
  if (overlaps(y, rows * groups * D * esize(prec), x, rows * D * esize(x_dt))) return PTDIT_ERR_ALIAS;
  return hip_status(gemm(prec, x, x_dt, rows, D, groups * D, w, b, nullptr, prec, y, prec, true, Ntok, heads, D,
                         PTDIT_K_GEMM_QKV, stream));
}

ptdit_status ptdit_window_attn(const void* qkv, const void* b_qkv, ptdit_dtype dt, ptdit_grid g, ptdit_win3 win,
                               ptdit_win3 shift, void* o, hipStream_t stream) {
  if (!valid_dtype(dt)) return PTDIT_ERR_DTYPE;
  ptdit_status st = check_grid(g);
  if (st) return st;
  if (win.t <= 0 || win.h <= 0 || win.w <= 0 || (int64_t)win.t * win.h * win.w > 128) return PTDIT_ERR_SHAPE;
  if (shift.t < 0 || shift.h < 0 || shift.w < 0 || shift.t >= win.t || shift.h >= win.h || shift.w >= win.w)
    return PTDIT_ERR_SHAPE;
  const int64_t N = (int64_t)g.F * g.H * g.W, rows = (int64_t)g.B * N;
  if (rows == 0) return PTDIT_OK;
  if (!qkv || !o) return PTDIT_ERR_NULL;
  if (!aligned16(qkv) || !aligned16(b_qkv) || !aligned16(o)) return PTDIT_ERR_ALIGN;
  const size_t es = esize(dt);
  if (overlaps(o, rows * g.D * es, qkv, rows * 3 * g.D * es) || overlaps(o, rows * g.D * es, b_qkv, 3 * g.D * es))
    return PTDIT_ERR_ALIAS;
  WindowDesc wd;
  wd.QKV = qkv; wd.bias_qkv = b_qkv; wd.O = o;
  wd.B = g.B; wd.F = g.F; wd.H = g.H; wd.W = g.W; wd.D = g.D; wd.heads = g.heads; wd.dh = g.D / g.heads;
  wd.wt = win.t; wd.wh = win.h; wd.ww = win.w;
  wd.st = shift.t; wd.sh = shift.h; wd.sw = shift.w;
  wd.Fp = (g.F + win.t - 1) / win.t * win.t;
  wd.Hp = (g.H + win.h - 1) / win.h * win.h;
  wd.Wp = (g.W + win.w - 1) / win.w * win.w;
  wd.scale = 1.0f / std::sqrt((float)wd.dh);
  TraceScope ts(PTDIT_K_ATTN_WINDOW, stream);
  return hip_status(launch_window(wd, dt == PTDIT_F32, stream));
}

size_t ptdit_attn_workspace_bytes(int32_t B, int32_t heads, int32_t Nk, ptdit_dtype dt) {
  if (B < 0 || heads <= 0 || Nk < 0 || !valid_dtype(dt)) return 0;
  return dt == PTDIT_BF16 ? flash_vt_bytes(B, heads, Nk) : 0;
}

ptdit_status ptdit_attn(const void* q, int64_t q_bstride, const void* k, const void* v, int64_t kv_bstride,
                        ptdit_dtype dt, int32_t B, int32_t heads, int32_t Nq, int32_t Nk, int32_t dh, void* o,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dt)) return PTDIT_ERR_DTYPE;
  if (B < 0 || heads <= 0 || Nq < 0 || Nk < 0 || (dh != 64 && dh != 72)) return PTDIT_ERR_SHAPE;
  if ((int64_t)B * heads > 65535 || Nq > (1 << 30) || (Nq > 0 && Nk == 0)) return PTDIT_ERR_SHAPE;
  if ((int64_t)B * Nq == 0) return PTDIT_OK;
  const int64_t hq = (int64_t)heads * Nq * dh, hk = (int64_t)heads * Nk * dh;
  if (q_bstride < hq || kv_bstride < hk) return PTDIT_ERR_SHAPE;
  if (!q || !k || !v || !o) return PTDIT_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(ws)) return PTDIT_ERR_ALIGN;
  const size_t need = ptdit_attn_workspace_bytes(B, heads, Nk, dt);
  if (need && (!ws || ws_bytes < need)) return PTDIT_ERR_WORKSPACE;
  const size_t es = esize(dt);
  const size_t qb = ((B - 1) * q_bstride + hq) * es, kb = ((B - 1) * kv_bstride + hk) * es;
  const size_t ob = (size_t)B * Nq * heads * dh * es;
  if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, kb) || overlaps(o, ob, ws, need) ||
      overlaps(ws, need, q, qb) || overlaps(ws, need, k, kb) || overlaps(ws, need, v, kb))
    return PTDIT_ERR_ALIAS;
  FlashDesc f;
  f.Q = q; f.q_bs = q_bstride; f.q_hs = (int64_t)Nq * dh;
  f.K = k; f.k_bs = kv_bstride; f.k_hs = (int64_t)Nk * dh;
  f.V = v; f.v_bs = kv_bstride; f.v_hs = (int64_t)Nk * dh;
  f.O = o; f.B = B; f.heads = heads; f.Nq = Nq; f.Nk = Nk; f.dh = dh; f.D = heads * dh;
  f.scale = 1.0f / std::sqrt((float)dh);
  if (need) { f.vt = ws; f.vt_bytes = need; }
  TraceScope ts(PTDIT_K_ATTN_FLASH, stream);
  return hip_status(launch_flash(f, dt == PTDIT_F32, stream));
}

ptdit_status ptdit_heads_to_tokens(const float* src, int32_t B, int32_t groups, int32_t heads, int32_t Ntok,
                                   int32_t dh, float* dst, hipStream_t stream) {
  if (B < 0 || groups < 1 || heads <= 0 || Ntok < 0 || dh <= 0 || dh % 4) return PTDIT_ERR_SHAPE;
  const int64_t n = (int64_t)B * groups * heads * Ntok * dh;
  if (n == 0) return PTDIT_OK;
  if ((int64_t)B * Ntok * groups * heads * dh / 4 > ((int64_t)1 << 40)) return PTDIT_ERR_SHAPE;
  if (!src || !dst) return PTDIT_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return PTDIT_ERR_ALIGN;
  if (overlaps(src, n * 4, dst, n * 4)) return PTDIT_ERR_ALIAS;
  return hip_status(launch_heads_to_tokens(src, dst, B, groups, heads, Ntok, dh, stream));
}

ptdit_status ptdit_f32_to_bf16(const float* src, int64_t n, void* dst, hipStream_t stream) {
  if (n < 0 || n % 8) return PTDIT_ERR_SHAPE;
  if (n == 0) return PTDIT_OK;
  if (!src || !dst) return PTDIT_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return PTDIT_ERR_ALIGN;
  if (overlaps(src, n * 4, dst, n * 2)) return PTDIT_ERR_ALIAS;
  return hip_status(launch_f32_to_bf16(src, (uint16_t*)dst, n, stream));
}

ptdit_status ptdit_add_f32(const float* a, const float* b, int64_t n, float* out, hipStream_t stream) {
  if (n < 0 || n % 4) return PTDIT_ERR_SHAPE;
  if (n == 0) return PTDIT_OK;
  if (!a || !b || !out) return PTDIT_ERR_NULL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return PTDIT_ERR_ALIGN;
  // out may be a or b exactly (element-wise), but not a shifted view of either
  const size_t nb = n * 4;
  if ((out != a && overlaps(out, nb, a, nb)) || (out != b && overlaps(out, nb, b, nb))) return PTDIT_ERR_ALIAS;
  return hip_status(launch_add_f32(a, b, out, n, stream));
}

// ------------------------------------------------------------------ calibration
ptdit_status ptdit_calibrate_mfma(int32_t blocks, int32_t iters, float* out, int64_t* flop, hipStream_t stream) {
  if (blocks <= 0 || blocks > 65535 || iters <= 0) return PTDIT_ERR_SHAPE;
  if (!out || !flop) return PTDIT_ERR_NULL;
  if (!aligned16(out)) return PTDIT_ERR_ALIGN;
  *flop = calib_mfma_flop(blocks, iters);
  return hip_status(launch_calib_mfma(blocks, iters, out, stream));
}

ptdit_status ptdit_calibrate_read(const void* buf, int64_t bytes, int32_t blocks, float* out, hipStream_t stream) {
  if (bytes <= 0 || bytes % 16 || blocks <= 0 || blocks > 65535) return PTDIT_ERR_SHAPE;
  if (!buf || !out) return PTDIT_ERR_NULL;
  if (!aligned16(buf) || !aligned16(out)) return PTDIT_ERR_ALIGN;
  if (overlaps(out, (size_t)blocks * 256 * 4, buf, (size_t)bytes)) return PTDIT_ERR_ALIAS;
  return hip_status(launch_calib_read(buf, bytes, blocks, out, stream));
}

ptdit_status ptdit_calibrate_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (bytes < 0 || bytes % 16) return PTDIT_ERR_SHAPE;
  if (bytes == 0) return PTDIT_OK;
  if (!src || !dst) return PTDIT_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return PTDIT_ERR_ALIGN;
  if (overlaps(dst, (size_t)bytes, src, (size_t)bytes)) return PTDIT_ERR_ALIAS;
  return hip_status(launch_calib_copy(src, dst, bytes, stream));
}

ptdit_status ptdit_proxy_pool_bwd(const float* d_proxies, ptdit_grid g, ptdit_win3 p, float* d_x,
                                  int32_t accumulate, hipStream_t stream) {
  if (g.B < 0 || g.F < 0 || g.H < 0 || g.W < 0 || g.D <= 0 || g.D % 4) return PTDIT_ERR_SHAPE;
  if (p.t <= 0 || p.h <= 0 || p.w <= 0) return PTDIT_ERR_SHAPE;
  if (g.F % p.t || g.H % p.h || g.W % p.w) return PTDIT_ERR_DIVISIBILITY;
  const int64_t N = (int64_t)g.F * g.H * g.W;
  // the kernel takes eight token rows per workgroup (a 32-bit grid)
  if (N > (int64_t)1 << 30 || (int64_t)g.B * N > (int64_t)INT32_MAX) return PTDIT_ERR_SHAPE;
  if ((int64_t)g.B * N == 0) return PTDIT_OK;
  if (!d_proxies || !d_x) return PTDIT_ERR_NULL;
  if (!aligned16(d_proxies) || !aligned16(d_x)) return PTDIT_ERR_ALIGN;
  const int64_t M = N / ((int64_t)p.t * p.h * p.w);
  if (overlaps(d_x, g.B * N * g.D * 4, d_proxies, g.B * M * g.D * 4)) return PTDIT_ERR_ALIAS;
  PoolBwdDesc d;
  d.dP = d_proxies; d.dx = d_x;
  d.B = g.B; d.F = g.F; d.H = g.H; d.W = g.W; d.D = g.D;
  d.pt = p.t; d.ph = p.h; d.pw = p.w;
  d.accumulate = accumulate != 0;
  TraceScope ts(PTDIT_K_BWD_POOL, stream);
  return hip_status(launch_pool_bwd(d, stream));
}

size_t ptdit_linear_bwd_workspace_bytes(int64_t rows, int32_t d_in, int32_t d_out) {
  if (rows < 0 || d_in <= 0 || d_out <= 0 || d_in % 8 || d_out % 8) return 0;
  int splits;
  int64_t tch;
  wgrad_plan(rows, d_in, d_out, splits, tch);
  const size_t ld = (size_t)splits * tch;
  return align_up((size_t)d_in * d_out * 2) + align_up((size_t)splits * d_out * d_in * 4) +
         align_up((size_t)colsum_splits(rows) * d_out * 4) + align_up(ld * d_out * 2) + align_up(ld * d_in * 2) +
         align_up((size_t)rows * d_out * 2);
}

static_assert(PTDIT_MAX_DW_GROUP <= GEMM_MAX_GROUPS, "one launch holds every product");

size_t ptdit_linear_bwd_dw_group_workspace_bytes(int32_t n, int64_t rows, int32_t d_in, int32_t d_out) {
  if (n < 1 || n > PTDIT_MAX_DW_GROUP || rows <= 0 || d_in <= 0 || d_out <= 0 || d_in % 8 || d_out % 8 ||
      !wgrad_token_major(rows, d_in, d_out, 0, 0))
    return 0;
  return wgrad_group_ws_bytes(n, rows, d_in, d_out);
}

ptdit_status ptdit_linear_bwd_dw_group(int32_t n, const void* const* x, const void* const* d_y, int64_t rows,
                                       int32_t d_in, int32_t d_out, float* const* d_w, float* const* d_b, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  if (n < 1 || n > PTDIT_MAX_DW_GROUP || rows < 0 || d_in <= 0 || d_out <= 0 || d_in % 8 || d_out % 8)
    return PTDIT_ERR_SHAPE;
  if (!x || !d_y || !d_w) return PTDIT_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!x[i] || !d_y[i] || !d_w[i]) return PTDIT_ERR_NULL;
  if (rows == 0) return PTDIT_OK;
  if (rows > (int64_t)65535 * 32 || !wgrad_token_major(rows, d_in, d_out, 0, 0)) return PTDIT_ERR_SHAPE;
  const size_t need = wgrad_group_ws_bytes(n, rows, d_in, d_out);
  if (!ws || ws_bytes < need) return PTDIT_ERR_WORKSPACE;
  if (!aligned16(ws)) return PTDIT_ERR_ALIGN;
  for (int i = 0; i < n; ++i)
    if (!aligned16(x[i]) || !aligned16(d_y[i]) || !aligned16(d_w[i]) || (d_b && !aligned16(d_b[i])))
      return PTDIT_ERR_ALIGN;
  const size_t xb = (size_t)rows * d_in * 2, yb = (size_t)rows * d_out * 2;
  const size_t wb = (size_t)d_out * d_in * 4, bb = (size_t)d_out * 4;
  for (int i = 0; i < n; ++i) {
    const void* outs[2] = {d_w[i], d_b ? d_b[i] : nullptr};
    const size_t osz[2] = {wb, bb};
    for (int o = 0; o < 2; ++o) {
      if (!outs[o]) continue;
      if (overlaps(outs[o], osz[o], ws, need)) return PTDIT_ERR_ALIAS;
      for (int j = 0; j < n; ++j) {
        if (overlaps(outs[o], osz[o], x[j], xb) || overlaps(outs[o], osz[o], d_y[j], yb)) return PTDIT_ERR_ALIAS;
        if (j != i && (overlaps(outs[o], osz[o], d_w[j], wb) || (d_b && overlaps(outs[o], osz[o], d_b[j], bb))))
          return PTDIT_ERR_ALIAS;
      }
    }
    if (d_b && overlaps(d_w[i], wb, d_b[i], bb)) return PTDIT_ERR_ALIAS;
    if (overlaps(ws, need, x[i], xb) || overlaps(ws, need, d_y[i], yb)) return PTDIT_ERR_ALIAS;
  }
  WgradGroupDesc d;
  d.n = n;
  for (int i = 0; i < n; ++i) {
    d.dy[i] = d_y[i];
    d.x[i] = x[i];
    d.dw[i] = d_w[i];
    d.db[i] = d_b ? d_b[i] : nullptr;
  }
  d.ws = ws;
  d.rows = rows; d.d_in = d_in; d.d_out = d_out;
  TraceScope ts(PTDIT_K_BWD_LINEAR, stream);
  return hip_status(launch_wgrad_group(d, stream));
}

ptdit_status ptdit_linear_bwd(const void* x, ptdit_dtype x_dt, int64_t rows, int32_t d_in, int32_t d_out,
                              const void* w, const void* d_y, ptdit_dtype dy_dt, float* d_x, float* d_w,
                              float* d_b, void* ws, size_t ws_bytes, hipStream_t stream) {
  return ptdit_linear_bwd_ex(x, x_dt, rows, d_in, d_out, w, d_y, dy_dt, d_x, nullptr, nullptr, d_w, d_b, ws,
                             ws_bytes, stream);
}

ptdit_status ptdit_linear_bwd_ex(const void* x, ptdit_dtype x_dt, int64_t rows, int32_t d_in, int32_t d_out,
                                 const void* w, const void* d_y, ptdit_dtype dy_dt, float* d_x,
                                 const float* d_x_add, uint16_t* d_x_bf16, float* d_w, float* d_b, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(x_dt) || !valid_dtype(dy_dt)) return PTDIT_ERR_DTYPE;
  if (rows < 0 || d_in <= 0 || d_out <= 0 || d_in % 8 || d_out % 8) return PTDIT_ERR_SHAPE;
  if (rows > (int64_t)65535 * 32 || (int64_t)d_in * d_out > ((int64_t)1 << 31)) return PTDIT_ERR_SHAPE;
  const bool want_dx = d_x || d_x_bf16;
  if (rows == 0 || (!want_dx && !d_w && !d_b)) return PTDIT_OK;
  if (!d_y || (d_w && !x) || (want_dx && !w)) return PTDIT_ERR_NULL;
  if (d_x_add && !d_x) return PTDIT_ERR_NULL;  // the sum is formed in fp32, so it needs d_x
  if (!aligned16(x) || !aligned16(w) || !aligned16(d_y) || !aligned16(d_x) || !aligned16(d_w) || !aligned16(d_b) ||
      !aligned16(ws) || !aligned16(d_x_add) || !aligned16(d_x_bf16))
    return PTDIT_ERR_ALIGN;
  const size_t need = ptdit_linear_bwd_workspace_bytes(rows, d_in, d_out);
  if (!ws || ws_bytes < need) return PTDIT_ERR_WORKSPACE;
  const size_t xb = (size_t)rows * d_in * esize(x_dt), yb = (size_t)rows * d_out * esize(dy_dt);
  const size_t wb = (size_t)d_out * d_in * 2, ab = (size_t)rows * d_in * 4;
  const void* outs[5] = {d_x, d_w, d_b, ws, d_x_bf16};
  const size_t osz[5] = {(size_t)rows * d_in * 4, (size_t)d_out * d_in * 4, (size_t)d_out * 4, need,
                         (size_t)rows * d_in * 2};
  for (int a = 0; a < 5; ++a) {
    if (overlaps(outs[a], osz[a], x, xb) || overlaps(outs[a], osz[a], d_y, yb) || overlaps(outs[a], osz[a], w, wb))
      return PTDIT_ERR_ALIAS;
    // the added gradient may be d_x itself (each element read, then written,
    // by the same lane of the same tile), else it overlaps no output
    if (!(a == 0 && d_x_add == d_x) && overlaps(outs[a], osz[a], d_x_add, ab)) return PTDIT_ERR_ALIAS;
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(outs[a], osz[a], outs[b], osz[b])) return PTDIT_ERR_ALIAS;
  }
  TraceScope ts(PTDIT_K_BWD_LINEAR, stream);
  char* wsp = (char*)ws;
  void* wt = wsp;
  float* part = (float*)(wsp + align_up((size_t)d_in * d_out * 2));
  int splits;
  int64_t tch;
  wgrad_plan(rows, d_in, d_out, splits, tch);
  const size_t ld = (size_t)splits * tch;
  float* dbp = (float*)((char*)part + align_up((size_t)splits * d_out * d_in * 4));
  uint16_t* dyt = (uint16_t*)((char*)dbp + align_up((size_t)colsum_splits(rows) * d_out * 4));
  uint16_t* xt = (uint16_t*)((char*)dyt + align_up(ld * d_out * 2));
  uint16_t* dyb = (uint16_t*)((char*)xt + align_up(ld * d_in * 2));
  WgradDesc d;
  d.dy = d_y; d.dy_f32 = dy_dt == PTDIT_F32;
  d.x = x; d.x_f32 = x_dt == PTDIT_F32;
  d.dyt = dyt; d.xt = xt;
  // with d_w, the transpose pass also leaves a bf16 copy of an fp32 d_y for d_x
  d.dyb = (want_dx && d_w && dy_dt == PTDIT_F32) ? dyb : nullptr;
  d.part = part; d.dbp = dbp; d.dw = d_w; d.db = d_b;
  d.rows = rows; d.d_in = d_in; d.d_out = d_out;
  if (d_w && !wgrad_token_major(rows, d_in, d_out, d.dy_f32, d.x_f32) && launch_wgrad_operands(d, stream) != hipSuccess)
    return PTDIT_ERR_HIP;
  if (want_dx) {
    // dX = dY W: with bf16 dY and d_out % 128 == 0 the ping-pong kernel reads
    // the weight as it lies (k-major: row o of W is k-slice row o); else the
    // projection kernels take a transposed copy. The added gradient is the
    // GEMM's residual, the bf16 copy its second output (or its only output
    // when d_x is NULL)
    GemmDesc g;
    g.A = d.dyb ? (const void*)d.dyb : d_y; g.a_f32 = !d.dyb && dy_dt == PTDIT_F32;
    const bool kmajor = !g.a_f32 && d_out % 128 == 0 && d_out >= 256 && rows >= 1024;
    if (kmajor) {
      g.w_kmajor = 1;
      g.ldw = d_in;
    } else {
      hipError_t e = launch_transpose_bf16(w, wt, d_out, d_in, stream);
      if (e != hipSuccess) return PTDIT_ERR_HIP;
    }
    g.W = kmajor ? w : wt; g.bias = nullptr;
    g.R = d_x_add; g.r_f32 = 1;
    g.Y = d_x ? (void*)d_x : (void*)d_x_bf16; g.y_f32 = d_x ? 1 : 0;
    g.Y2 = d_x ? d_x_bf16 : nullptr;
    g.M = rows; g.N = d_in; g.K = d_out;
    g.head_major = false; g.Ntok = rows; g.heads = 0; g.dh = 0; g.D = d_in;
    g.act = 0;
    if (launch_gemm_bf16(g, stream) != hipSuccess) return PTDIT_ERR_HIP;
  }
  if ((d_w || d_b) && launch_wgrad(d, stream) != hipSuccess) return PTDIT_ERR_HIP;
  return PTDIT_OK;
}

ptdit_status ptdit_trace_enable(int32_t kernel_class, int32_t capacity) {
  ptdit_trace_disable();
  if (capacity <= 0 || kernel_class < 0) return PTDIT_ERR_SHAPE;
  g_trace.start.resize(capacity);
  g_trace.stop.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    // no system-scope fence: the events only time work on this device
    if (hipEventCreateWithFlags(&g_trace.start[i], hipEventDisableSystemFence) != hipSuccess ||
        hipEventCreateWithFlags(&g_trace.stop[i], hipEventDisableSystemFence) != hipSuccess) {
      g_trace.start.resize(i);
      g_trace.stop.resize(i);
      ptdit_trace_disable();
      return PTDIT_ERR_HIP;
    }
  }
  g_trace.cls = kernel_class;
  g_trace.cap = capacity;
  g_trace.count = 0;
  return PTDIT_OK;
}

int32_t ptdit_trace_read(float* ms, int32_t max) {
  int n = 0;
  for (int i = 0; i < g_trace.count && i < max; ++i) {
    if (hipEventSynchronize(g_trace.stop[i]) != hipSuccess) break;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_trace.start[i], g_trace.stop[i]) != hipSuccess) break;
    ms[n++] = t;
  }
  return n;
}

void ptdit_trace_disable(void) {
  for (size_t i = 0; i < g_trace.start.size(); ++i) (void)hipEventDestroy(g_trace.start[i]);
  for (size_t i = 0; i < g_trace.stop.size(); ++i) (void)hipEventDestroy(g_trace.stop[i]);
  g_trace.start.clear();
  g_trace.stop.clear();
  g_trace.cls = -1;
  g_trace.cap = 0;
  g_trace.count = 0;
}

}  // extern "C"
