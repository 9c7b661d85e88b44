// arn_pyext.cpp -- the Python binding's per-call argument marshalling, in
// C++ (the module residual_add_rmsnorm_amd.lib._native).
//
// Each function takes torch tensors, checks them, reduces them to the
// (device pointer, row stride) pairs of the C ABI in include/arn.h and
// calls the entry point of the same name on the current stream of the
// tensors' device.  Nothing of the operator is computed here: every step
// runs in libarn.so's kernels.  Doing these checks in Python costs several
// microseconds per call (each tensor attribute is a Python-level lookup),
// which is more than a decode-sized kernel takes on the GPU; here they cost
// a fraction of a microsecond.
//
// Layout rules are those of the vLLM API page "vllm.kernels.aiter_ops"
// (flatten_to_2d_is_free): the last dimension has unit stride and the
// leading dimensions flatten to rows of one uniform pitch without a copy.
// A padded pitch is accepted; a layout that would need a copy raises
// ValueError and is never copied.
//
// The entry points are reached through addresses that the Python loader
// takes from its ctypes handle of libarn.so (bind()), so this module and
// ctypes share one copy of the library and of its per-thread tuning state.
//
// The same functions back the torch custom ops of a decode step (arn::*,
// registered below for the CUDA dispatch key), so a call through torch.ops
// reaches the C ABI without entering Python; their fake implementations
// (output shapes for the compiler) are registered from Python.
#include <torch/extension.h>

#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPStream.h>

#include <string>

#include "arn.h"

namespace py = pybind11;

namespace {

struct Entry {
  decltype(&arn_rmsnorm) rmsnorm = nullptr;
  decltype(&arn_fused_add_rmsnorm) fused_add_rmsnorm = nullptr;
  decltype(&arn_rmsnorm_fp8) rmsnorm_fp8 = nullptr;
  decltype(&arn_fused_add_rmsnorm_fp8) fused_add_rmsnorm_fp8 = nullptr;
  decltype(&arn_norm) norm = nullptr;
  decltype(&arn_silu_and_mul) silu_and_mul = nullptr;
  decltype(&arn_silu_and_mul_fp8) silu_and_mul_fp8 = nullptr;
  decltype(&arn_fp8_gemm) fp8_gemm = nullptr;
  decltype(&arn_fp8_gemm_ws) fp8_gemm_ws = nullptr;
  decltype(&arn_fp8_gemm_preshuffled) fp8_gemm_preshuffled = nullptr;
  decltype(&arn_fp8_gemm_preshuffled_ws) fp8_gemm_preshuffled_ws = nullptr;
  decltype(&arn_fp8_gemm_preshuffled_noalloc) fp8_gemm_preshuffled_noalloc = nullptr;
  decltype(&arn_fp8_weight_preshuffled_bytes) fp8_weight_preshuffled_bytes = nullptr;
  decltype(&arn_status_str) status_str = nullptr;
};
Entry g_entry;
bool g_bound = false;
// _lib.check(status, name): raises the package's ArnError.  Held for the
// life of the process (never destroyed after the interpreter is gone).
py::object* g_check = nullptr;

template <typename F>
void take(const py::dict& addrs, const char* name, F& fn) {
  if (!addrs.contains(name)) throw py::value_error(std::string("bind: no address for ") + name);
  const uintptr_t p = addrs[name].cast<uintptr_t>();
  if (p == 0) throw py::value_error(std::string("bind: null address for ") + name);
  fn = reinterpret_cast<F>(p);
}

void bind(const py::dict& addrs, const py::object& check) {
  Entry e;
  take(addrs, "arn_rmsnorm", e.rmsnorm);
  take(addrs, "arn_fused_add_rmsnorm", e.fused_add_rmsnorm);
  take(addrs, "arn_rmsnorm_fp8", e.rmsnorm_fp8);
  take(addrs, "arn_fused_add_rmsnorm_fp8", e.fused_add_rmsnorm_fp8);
  take(addrs, "arn_norm", e.norm);
  take(addrs, "arn_silu_and_mul", e.silu_and_mul);
  take(addrs, "arn_silu_and_mul_fp8", e.silu_and_mul_fp8);
  take(addrs, "arn_fp8_gemm", e.fp8_gemm);
  take(addrs, "arn_fp8_gemm_ws", e.fp8_gemm_ws);
  take(addrs, "arn_fp8_gemm_preshuffled", e.fp8_gemm_preshuffled);
  take(addrs, "arn_fp8_gemm_preshuffled_ws", e.fp8_gemm_preshuffled_ws);
  take(addrs, "arn_fp8_gemm_preshuffled_noalloc", e.fp8_gemm_preshuffled_noalloc);
  take(addrs, "arn_fp8_weight_preshuffled_bytes", e.fp8_weight_preshuffled_bytes);
  take(addrs, "arn_status_str", e.status_str);
  g_entry = e;
  if (g_check == nullptr) g_check = new py::object(check);
  g_bound = true;
}

const Entry& entry() {
  TORCH_CHECK(g_bound, "libarn.so entry points not bound (load the package's binding first)");
  return g_entry;
}

// A nonzero status from the C ABI.  The functions below touch no Python
// object (a torch op runs them without the interpreter lock); the Python
// wrappers turn this into the package's ArnError and the torch ops into a
// RuntimeError.
struct AbiStatus {
  int status;
  const char* name;
};

void check(int status, const char* name) {
  if (status != ARN_OK) throw AbiStatus{status, name};
}

// A refused argument: ValueError in Python, from either path.
[[noreturn]] void refuse(const std::string& msg) { TORCH_CHECK_VALUE(false, msg); }

std::string dtype_name(at::ScalarType t) {
  switch (t) {
    case at::kBFloat16: return "torch.bfloat16";
    case at::kHalf: return "torch.float16";
    case at::kFloat: return "torch.float32";
    case at::kFloat8_e4m3fn: return "torch.float8_e4m3fn";
    default: return std::string("torch.") + c10::toString(t);
  }
}

int dtype_code(at::ScalarType t) {
  if (t == at::kBFloat16) return ARN_BF16;
  if (t == at::kHalf) return ARN_FP16;
  return -1;
}

struct RowView {
  int64_t rows, hidden, stride;
};

// (rows, hidden, row stride) of a tensor viewed as 2-D rows without a
// copy: the leading dimensions, skipping those of size 1, must step by one
// pitch times the product of the sizes inside them.
RowView row_view(const at::Tensor& t, const char* name) {
  const int64_t nd = t.dim();
  if (nd == 0) refuse(std::string(name) + ": needs at least one dimension");
  const int64_t hidden = t.size(nd - 1);
  if (hidden > 0 && t.is_contiguous()) return {t.numel() / hidden, hidden, hidden};
  if (hidden > 1 && t.stride(nd - 1) != 1) refuse(std::string(name) + ": last dimension must have unit stride");
  int64_t rows = 1;
  for (int64_t i = 0; i + 1 < nd; ++i) rows *= t.size(i);
  int64_t pitch = -1, expected = 0;
  for (int64_t i = nd - 2; i >= 0; --i) {
    const int64_t n = t.size(i);
    if (n == 1) continue;
    if (pitch < 0) {
      pitch = t.stride(i);
      expected = pitch * n;
    } else {
      if (t.stride(i) != expected) {
        refuse(std::string(name) + ": leading dims do not flatten to one row pitch without a copy");
      }
      expected *= n;
    }
  }
  if (pitch < 0) pitch = hidden;
  if (rows > 1 && pitch < hidden) {
    refuse(std::string(name) + ": rows overlap (row stride " + std::to_string(pitch) +
           " < hidden " + std::to_string(hidden) + ")");
  }
  return {rows, hidden, pitch};
}

void need_gpu(const at::Tensor& x) {
  if (!x.is_cuda()) refuse("tensors must live on a GPU device");
}

int act_dtype(const at::Tensor& x) {
  const int dt = dtype_code(x.scalar_type());
  if (dt < 0) refuse("activations must be bfloat16 or float16, got " + dtype_name(x.scalar_type()));
  return dt;
}

void same_as_x(const at::Tensor& r, const at::Tensor& x, const char* msg) {
  if (r.scalar_type() != x.scalar_type() || !r.sizes().equals(x.sizes()) || r.device() != x.device()) {
    refuse(msg);
  }
}

const void* weight_ptr(const c10::optional<at::Tensor>& w, const at::Tensor& x, int64_t hidden) {
  if (!w.has_value()) return nullptr;
  const at::Tensor& t = *w;
  if (t.scalar_type() != x.scalar_type()) refuse("weight dtype must match x dtype");
  if (t.dim() != 1 || t.size(0) != hidden || (hidden > 1 && t.stride(0) != 1)) {
    refuse("weight must be a contiguous vector of " + std::to_string(hidden) + " elements");
  }
  if (t.device() != x.device()) refuse("weight must be on x's device");
  return t.data_ptr();
}

at::Tensor out_like(const at::Tensor& x, const c10::optional<at::Tensor>& out, at::ScalarType dt) {
  if (!out.has_value()) return at::empty(x.sizes(), x.options().dtype(dt));
  const at::Tensor& o = *out;
  if (!o.sizes().equals(x.sizes()) || o.scalar_type() != dt || o.device() != x.device()) {
    refuse("out must have x's shape and dtype " + dtype_name(dt) + " on x's device");
  }
  return o;
}

// The FP8 scale operand: the static dequant scale (one fp32 value, read),
// or the dynamic per-row scales (rows fp32 values, written; allocated when
// not given).
at::Tensor fp8_scale(const at::Tensor& x, int64_t rows, const c10::optional<at::Tensor>& scale,
                     bool dynamic, const c10::optional<at::Tensor>& scales_out) {
  if (dynamic) {
    at::Tensor s;
    if (scales_out.has_value()) {
      s = *scales_out;
    } else if (x.dim() > 1) {
      s = at::empty(x.sizes().slice(0, x.dim() - 1), x.options().dtype(at::kFloat));
    } else {
      s = at::empty({1}, x.options().dtype(at::kFloat));
    }
    if (s.scalar_type() != at::kFloat || s.numel() != rows || !s.is_contiguous() ||
        s.device() != x.device()) {
      refuse("scales_out must be " + std::to_string(rows) +
             " contiguous float32 values on x's device");
    }
    return s;
  }
  if (!scale.has_value()) refuse("static FP8 needs `scale` (one float32 dequant scale on the device)");
  const at::Tensor& s = *scale;
  if (s.scalar_type() != at::kFloat || s.numel() != 1 || s.device() != x.device()) {
    refuse("scale must be one float32 value on x's device");
  }
  return s;
}

// x's device made current for the call, and its current stream.
struct OnDevice {
  c10::DeviceGuard guard;
  hipStream_t stream;
  explicit OnDevice(const at::Tensor& x)
      : guard(x.device()), stream(c10::hip::getCurrentHIPStream(x.device().index()).stream()) {}
};

py::tuple py_row_view(const at::Tensor& t, const std::string& name) {
  const RowView v = row_view(t, name.c_str());
  return py::make_tuple(v.rows, v.hidden, v.stride);
}

// ---------------------------------------------------------------------------
// The norm forms (arn_rmsnorm, arn_fused_add_rmsnorm, arn_rmsnorm_fp8,
// arn_fused_add_rmsnorm_fp8, arn_norm).
// ---------------------------------------------------------------------------
at::Tensor rmsnorm(const at::Tensor& x, const c10::optional<at::Tensor>& weight, double eps,
                   const c10::optional<at::Tensor>& out_in) {
  const Entry& e = entry();
  need_gpu(x);
  const int dt = act_dtype(x);
  const RowView xv = row_view(x, "x");
  at::Tensor out = out_like(x, out_in, x.scalar_type());
  const RowView ov = row_view(out, "out");
  const void* wp = weight_ptr(weight, x, xv.hidden);
  int st;
  {
    OnDevice on(x);
    st = e.rmsnorm(out.data_ptr(), ov.stride, x.data_ptr(), xv.stride, wp, (float)eps, xv.rows,
                   xv.hidden, dt, on.stream);
  }
  check(st, "arn_rmsnorm");
  return out;
}

at::Tensor fused_add_rmsnorm(const at::Tensor& x, const at::Tensor& residual,
                             const c10::optional<at::Tensor>& weight, double eps,
                             const c10::optional<at::Tensor>& out_in) {
  const Entry& e = entry();
  need_gpu(x);
  const int dt = act_dtype(x);
  same_as_x(residual, x, "residual must match x in shape, dtype and device");
  const RowView xv = row_view(x, "x");
  const RowView rv = row_view(residual, "residual");
  at::Tensor out = out_like(x, out_in, x.scalar_type());
  const RowView ov = row_view(out, "out");
  const void* wp = weight_ptr(weight, x, xv.hidden);
  int st;
  {
    OnDevice on(x);
    st = e.fused_add_rmsnorm(out.data_ptr(), ov.stride, x.data_ptr(), xv.stride, residual.data_ptr(),
                             rv.stride, wp, (float)eps, xv.rows, xv.hidden, dt, on.stream);
  }
  check(st, "arn_fused_add_rmsnorm");
  return out;
}

using Pair = std::tuple<at::Tensor, at::Tensor>;

Pair rmsnorm_fp8(const at::Tensor& x, const c10::optional<at::Tensor>& weight, double eps,
                 const c10::optional<at::Tensor>& scale, bool dynamic,
                 const c10::optional<at::Tensor>& out_in,
                 const c10::optional<at::Tensor>& scales_out) {
  const Entry& e = entry();
  need_gpu(x);
  const int dt = act_dtype(x);
  const RowView xv = row_view(x, "x");
  at::Tensor out = out_like(x, out_in, at::kFloat8_e4m3fn);
  const RowView ov = row_view(out, "out");
  const void* wp = weight_ptr(weight, x, xv.hidden);
  at::Tensor sc = fp8_scale(x, xv.rows, scale, dynamic, scales_out);
  int st;
  {
    OnDevice on(x);
    st = e.rmsnorm_fp8(static_cast<uint8_t*>(out.data_ptr()), ov.stride,
                       static_cast<float*>(sc.data_ptr()), dynamic ? ARN_FP8_DYNAMIC : ARN_FP8_STATIC,
                       x.data_ptr(), xv.stride, wp, (float)eps, xv.rows, xv.hidden, dt, on.stream);
  }
  check(st, "arn_rmsnorm_fp8");
  return {out, sc};
}

Pair fused_add_rmsnorm_fp8(const at::Tensor& x, const at::Tensor& residual,
                           const c10::optional<at::Tensor>& weight, double eps,
                           const c10::optional<at::Tensor>& scale, bool dynamic,
                           const c10::optional<at::Tensor>& out_in,
                           const c10::optional<at::Tensor>& scales_out) {
  const Entry& e = entry();
  need_gpu(x);
  const int dt = act_dtype(x);
  same_as_x(residual, x, "residual must match x in shape, dtype and device");
  const RowView xv = row_view(x, "x");
  const RowView rv = row_view(residual, "residual");
  at::Tensor out = out_like(x, out_in, at::kFloat8_e4m3fn);
  const RowView ov = row_view(out, "out");
  const void* wp = weight_ptr(weight, x, xv.hidden);
  at::Tensor sc = fp8_scale(x, xv.rows, scale, dynamic, scales_out);
  int st;
  {
    OnDevice on(x);
    st = e.fused_add_rmsnorm_fp8(static_cast<uint8_t*>(out.data_ptr()), ov.stride,
                                 static_cast<float*>(sc.data_ptr()),
                                 dynamic ? ARN_FP8_DYNAMIC : ARN_FP8_STATIC, x.data_ptr(), xv.stride,
                                 residual.data_ptr(), rv.stride, wp, (float)eps, xv.rows, xv.hidden,
                                 dt, on.stream);
  }
  check(st, "arn_fused_add_rmsnorm_fp8");
  return {out, sc};
}

// fp8: "" (16-bit out), "static" or "dynamic".  Returns (out, scale
// tensor); the scale is undefined for a 16-bit output.
Pair norm(const at::Tensor& x, const c10::optional<at::Tensor>& weight, double eps,
          const c10::optional<at::Tensor>& residual, int64_t variance_size, const std::string& fp8,
          const c10::optional<at::Tensor>& scale, const c10::optional<at::Tensor>& out_in,
          const c10::optional<at::Tensor>& scales_out) {
  const Entry& e = entry();
  need_gpu(x);
  const int dt = act_dtype(x);
  const RowView xv = row_view(x, "x");
  int64_t rs = 0;
  if (residual.has_value()) {
    same_as_x(*residual, x, "residual must match x in shape, dtype and device");
    rs = row_view(*residual, "residual").stride;
  }
  at::Tensor out = out_like(x, out_in, fp8.empty() ? x.scalar_type() : at::kFloat8_e4m3fn);
  const RowView ov = row_view(out, "out");
  const void* wp = weight_ptr(weight, x, xv.hidden);
  at::Tensor sc;
  int fmt = 0;  // 16-bit out
  if (!fp8.empty()) {
    if (fp8 != "static" && fp8 != "dynamic") refuse("fp8 must be None, 'static' or 'dynamic'");
    sc = fp8_scale(x, xv.rows, scale, fp8 == "dynamic", scales_out);
    fmt = fp8 == "dynamic" ? 2 : 1;
  }
  int st;
  {
    OnDevice on(x);
    arn_norm_args a;
    a.struct_size = sizeof(arn_norm_args);
    a.dtype = dt;
    a.out_format = fmt;
    a.out = out.data_ptr();
    a.out_stride = ov.stride;
    a.scale = sc.defined() ? static_cast<float*>(sc.data_ptr()) : nullptr;
    a.x = x.data_ptr();
    a.x_stride = xv.stride;
    a.residual = residual.has_value() ? residual->data_ptr() : nullptr;
    a.residual_stride = rs;
    a.weight = wp;
    a.eps = (float)eps;
    a.rows = xv.rows;
    a.hidden = xv.hidden;
    a.variance_size = variance_size;
    a.stream = on.stream;
    st = e.norm(&a);
  }
  check(st, "arn_norm");
  return {out, sc};
}

// ---------------------------------------------------------------------------
// SwiGLU of a [..., 2d] gate|up tensor (arn_silu_and_mul, arn_silu_and_mul_fp8).
// ---------------------------------------------------------------------------
RowView glu_view(const at::Tensor& x) {
  need_gpu(x);
  act_dtype(x);
  const RowView v = row_view(x, "x");
  if (v.hidden % 2) refuse("the last dimension of x must be 2*d (gate | up)");
  return v;  // hidden holds 2d
}

at::Tensor glu_out(const at::Tensor& x, const c10::optional<at::Tensor>& out, at::ScalarType dt,
                   int64_t d) {
  std::vector<int64_t> shape(x.sizes().begin(), x.sizes().end());
  shape.back() = d;
  if (!out.has_value()) return at::empty(shape, x.options().dtype(dt));
  const at::Tensor& o = *out;
  if (!o.sizes().equals(shape) || o.scalar_type() != dt || o.device() != x.device()) {
    std::string s = "(";
    for (size_t i = 0; i < shape.size(); ++i) s += (i ? ", " : "") + std::to_string(shape[i]);
    s += shape.size() == 1 ? ",)" : ")";
    refuse("out must have shape " + s + " and dtype " + dtype_name(dt) + " on x's device");
  }
  return o;
}

at::Tensor silu_and_mul(const at::Tensor& x, const c10::optional<at::Tensor>& out_in) {
  const Entry& e = entry();
  const RowView xv = glu_view(x);
  const int64_t d = xv.hidden / 2;
  at::Tensor out = glu_out(x, out_in, x.scalar_type(), d);
  const RowView ov = row_view(out, "out");
  const char* base = static_cast<const char*>(x.data_ptr());
  int st;
  {
    OnDevice on(x);
    st = e.silu_and_mul(out.data_ptr(), ov.stride, base, xv.stride, base + 2 * d, xv.stride,
                        xv.rows, d, dtype_code(x.scalar_type()), on.stream);
  }
  check(st, "arn_silu_and_mul");
  return out;
}

Pair silu_and_mul_fp8(const at::Tensor& x, const c10::optional<at::Tensor>& scale, bool dynamic,
                      const c10::optional<at::Tensor>& out_in,
                      const c10::optional<at::Tensor>& scales_out) {
  const Entry& e = entry();
  const RowView xv = glu_view(x);
  const int64_t d = xv.hidden / 2;
  at::Tensor out = glu_out(x, out_in, at::kFloat8_e4m3fn, d);
  const RowView ov = row_view(out, "out");
  at::Tensor sc = fp8_scale(x, xv.rows, scale, dynamic, scales_out);
  const char* base = static_cast<const char*>(x.data_ptr());
  int st;
  {
    OnDevice on(x);
    st = e.silu_and_mul_fp8(static_cast<uint8_t*>(out.data_ptr()), ov.stride,
                            static_cast<float*>(sc.data_ptr()),
                            dynamic ? ARN_FP8_DYNAMIC : ARN_FP8_STATIC, base, xv.stride,
                            base + 2 * d, xv.stride, xv.rows, d, dtype_code(x.scalar_type()),
                            on.stream);
  }
  check(st, "arn_silu_and_mul_fp8");
  return {out, sc};
}

// ---------------------------------------------------------------------------
// The e4m3 GEMM (arn_fp8_gemm[_ws], arn_fp8_gemm_preshuffled[_ws|_noalloc]).
// ---------------------------------------------------------------------------
void fp8_matrix(const at::Tensor& t, const char* name) {
  need_gpu(t);
  const auto st = t.scalar_type();
  if ((st != at::kFloat8_e4m3fn && st != at::kByte) || t.dim() != 2 || t.stride(1) != 1) {
    refuse(std::string(name) + " must be a 2-D e4m3 (or uint8) tensor with unit column stride");
  }
}

void gemm_scale(const at::Tensor& s, int64_t cnt, const at::Tensor& a, const char* name) {
  if (s.scalar_type() != at::kFloat || !s.is_contiguous() || (s.numel() != 1 && s.numel() != cnt) ||
      s.device() != a.device()) {
    refuse(std::string(name) + " must hold 1 or " + std::to_string(cnt) + " contiguous float32 values");
  }
}

at::Tensor gemm_out(const at::Tensor& a, int64_t m, int64_t n, int out_code,
                    const c10::optional<at::Tensor>& out_in) {
  at::Tensor out;
  if (out_in.has_value()) {
    out = *out_in;
  } else {
    if (out_code < 0) refuse("out must be [M, N] bfloat16/float16 with unit column stride");
    out = at::empty({m, n}, a.options().dtype(out_code == ARN_BF16 ? at::kBFloat16 : at::kHalf));
  }
  if (out.dim() != 2 || out.size(0) != m || out.size(1) != n || dtype_code(out.scalar_type()) < 0 ||
      out.stride(1) != 1) {
    refuse("out must be [M, N] bfloat16/float16 with unit column stride");
  }
  return out;
}

// b: the row-major weight [N, K], or with pre_n >= 0 the pre-shuffled
// bytes of an N x K weight (pre_n = N, pre_k = K).  out_code: the output
// dtype's ABI code for an allocated out (-1: not a served dtype).
at::Tensor fp8_gemm(const at::Tensor& a, const at::Tensor& scale_a, const at::Tensor& b,
                    const at::Tensor& scale_b, int out_code, const c10::optional<at::Tensor>& out_in,
                    const c10::optional<at::Tensor>& workspace, int64_t pre_n, int64_t pre_k) {
  const Entry& e = entry();
  const bool pre = pre_n >= 0;
  fp8_matrix(a, "a");
  if (!pre) fp8_matrix(b, "b");
  if (b.device() != a.device()) refuse("a and b must be on the same device");
  const int64_t m = a.size(0), k = a.size(1);
  const int64_t n = pre ? pre_n : b.size(0);
  const int64_t kb = pre ? pre_k : b.size(1);
  if (kb != k) refuse("a and b must have the same K");
  if (pre && b.numel() * b.element_size() < e.fp8_weight_preshuffled_bytes(n, k)) {
    refuse("b_shuffled is smaller than a pre-shuffled n x k weight");
  }
  gemm_scale(scale_a, m, a, "scale_a");
  gemm_scale(scale_b, n, a, "scale_b");
  at::Tensor out = gemm_out(a, m, n, out_code, out_in);
  const int a_rows = (scale_a.numel() > 1 || m == 1) ? 1 : 0;
  const int b_rows = (scale_b.numel() > 1 || n == 1) ? 1 : 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (workspace.has_value()) {
    const at::Tensor& w = *workspace;
    if (w.device() != a.device() || !w.is_contiguous()) {
      refuse("workspace must be a contiguous tensor on a's device");
    }
    ws = w.data_ptr();
    ws_bytes = (size_t)w.numel() * (size_t)w.element_size();
  }
  const int oc = dtype_code(out.scalar_type());
  const auto* ap = static_cast<const uint8_t*>(a.data_ptr());
  const auto* bp = static_cast<const uint8_t*>(b.data_ptr());
  const auto* sa = static_cast<const float*>(scale_a.data_ptr());
  const auto* sb = static_cast<const float*>(scale_b.data_ptr());
  const char* name;
  int st;
  {
    OnDevice on(a);
    if (pre && ws) {
      name = "arn_fp8_gemm_preshuffled_ws";
      st = e.fp8_gemm_preshuffled_ws(out.data_ptr(), out.stride(0), oc, ap, a.stride(0), sa, a_rows,
                                     bp, sb, b_rows, m, n, k, ws, ws_bytes, on.stream);
    } else if (pre) {
      name = "arn_fp8_gemm_preshuffled";
      st = e.fp8_gemm_preshuffled(out.data_ptr(), out.stride(0), oc, ap, a.stride(0), sa, a_rows, bp,
                                  sb, b_rows, m, n, k, on.stream);
    } else if (ws) {
      name = "arn_fp8_gemm_ws";
      st = e.fp8_gemm_ws(out.data_ptr(), out.stride(0), oc, ap, a.stride(0), sa, a_rows, bp,
                         b.stride(0), sb, b_rows, m, n, k, ws, ws_bytes, on.stream);
    } else {
      name = "arn_fp8_gemm";
      st = e.fp8_gemm(out.data_ptr(), out.stride(0), oc, ap, a.stride(0), sa, a_rows, bp,
                      b.stride(0), sb, b_rows, m, n, k, on.stream);
    }
  }
  check(st, name);
  return out;
}

at::Tensor fp8_gemm_preshuffled_noalloc(const at::Tensor& a, const at::Tensor& scale_a,
                                        const at::Tensor& b, int64_t n, int64_t kb,
                                        const at::Tensor& scale_b, int out_code,
                                        const c10::optional<at::Tensor>& out_in) {
  const Entry& e = entry();
  fp8_matrix(a, "a");
  if (b.device() != a.device()) refuse("a and b must be on the same device");
  const int64_t m = a.size(0), k = a.size(1);
  if (kb != k) refuse("a and b must have the same K");
  gemm_scale(scale_a, m, a, "scale_a");
  gemm_scale(scale_b, n, a, "scale_b");
  at::Tensor out = gemm_out(a, m, n, out_code, out_in);
  int st;
  {
    OnDevice on(a);
    st = e.fp8_gemm_preshuffled_noalloc(
        out.data_ptr(), out.stride(0), dtype_code(out.scalar_type()),
        static_cast<const uint8_t*>(a.data_ptr()), a.stride(0),
        static_cast<const float*>(scale_a.data_ptr()), (scale_a.numel() > 1 || m == 1) ? 1 : 0,
        static_cast<const uint8_t*>(b.data_ptr()), static_cast<const float*>(scale_b.data_ptr()),
        (scale_b.numel() > 1 || n == 1) ? 1 : 0, m, n, k, on.stream);
  }
  check(st, "arn_fp8_gemm_preshuffled_noalloc");
  return out;
}

// ---------------------------------------------------------------------------
// Python entry points.  The checks and the launch run without the
// interpreter lock (as a ctypes call or a torch op would), so other Python
// threads keep running during the launch; a status from the C ABI then
// becomes the package's ArnError (raised by _lib.check, lock held again).
// ---------------------------------------------------------------------------
template <typename F>
auto from_python(F&& f) -> decltype(f()) {
  try {
    py::gil_scoped_release unlocked;
    return f();
  } catch (const AbiStatus& e) {
    (*g_check)(e.status, e.name);
    throw std::runtime_error(std::string(e.name) + ": status " + std::to_string(e.status));
  }
}

// ---------------------------------------------------------------------------
// torch custom ops (CUDA kernels of the arn:: schemas below): a status from
// the C ABI becomes a RuntimeError naming the entry point and the status.
// ---------------------------------------------------------------------------
template <typename F>
auto from_torch(F&& f) -> decltype(f()) {
  try {
    return f();
  } catch (const AbiStatus& e) {
    TORCH_CHECK(false, e.name, ": ", entry().status_str(e.status), " (status ", e.status, ")");
  }
}

using OptT = c10::optional<at::Tensor>;

at::Tensor op_rmsnorm(const at::Tensor& x, const OptT& w, double eps) {
  return from_torch([&] { return rmsnorm(x, w, eps, c10::nullopt); });
}
at::Tensor op_fused_add_rmsnorm(const at::Tensor& x, at::Tensor& residual, const OptT& w,
                                double eps) {
  return from_torch([&] { return fused_add_rmsnorm(x, residual, w, eps, c10::nullopt); });
}
at::Tensor op_rmsnorm_fp8_static(const at::Tensor& x, const OptT& w, double eps,
                                 const at::Tensor& scale) {
  return from_torch([&] {
    return std::get<0>(rmsnorm_fp8(x, w, eps, scale, false, c10::nullopt, c10::nullopt));
  });
}
Pair op_rmsnorm_fp8_dynamic(const at::Tensor& x, const OptT& w, double eps) {
  return from_torch([&] { return rmsnorm_fp8(x, w, eps, c10::nullopt, true, c10::nullopt, c10::nullopt); });
}
at::Tensor op_fused_add_rmsnorm_fp8_static(const at::Tensor& x, at::Tensor& residual, const OptT& w,
                                           double eps, const at::Tensor& scale) {
  return from_torch([&] {
    return std::get<0>(
        fused_add_rmsnorm_fp8(x, residual, w, eps, scale, false, c10::nullopt, c10::nullopt));
  });
}
Pair op_fused_add_rmsnorm_fp8_dynamic(const at::Tensor& x, at::Tensor& residual, const OptT& w,
                                      double eps) {
  return from_torch([&] {
    return fused_add_rmsnorm_fp8(x, residual, w, eps, c10::nullopt, true, c10::nullopt, c10::nullopt);
  });
}
at::Tensor op_silu_and_mul(const at::Tensor& x) {
  return from_torch([&] { return silu_and_mul(x, c10::nullopt); });
}
at::Tensor op_silu_and_mul_fp8_static(const at::Tensor& x, const at::Tensor& scale) {
  return from_torch(
      [&] { return std::get<0>(silu_and_mul_fp8(x, scale, false, c10::nullopt, c10::nullopt)); });
}
Pair op_silu_and_mul_fp8_dynamic(const at::Tensor& x) {
  return from_torch([&] { return silu_and_mul_fp8(x, c10::nullopt, true, c10::nullopt, c10::nullopt); });
}
int out_code_of(const c10::optional<at::ScalarType>& dt) {
  return dt.has_value() ? dtype_code(*dt) : ARN_BF16;
}
at::Tensor op_fp8_gemm(const at::Tensor& a, const at::Tensor& scale_a, const at::Tensor& b,
                       const at::Tensor& scale_b, c10::optional<at::ScalarType> out_dtype) {
  return from_torch([&] {
    return fp8_gemm(a, scale_a, b, scale_b, out_code_of(out_dtype), c10::nullopt, c10::nullopt, -1, -1);
  });
}
at::Tensor op_fp8_gemm_preshuffled(const at::Tensor& a, const at::Tensor& scale_a,
                                   const at::Tensor& b_shuffled, int64_t n, int64_t k,
                                   const at::Tensor& scale_b, c10::optional<at::ScalarType> out_dtype) {
  return from_torch([&] {
    if (n < 0 || k <= 0) refuse("n must be >= 0 and k >= 1");
    return fp8_gemm(a, scale_a, b_shuffled, scale_b, out_code_of(out_dtype), c10::nullopt,
                    c10::nullopt, n, k);
  });
}

}  // namespace

// The ops of a decode step, in the arn namespace (the Python module adds the
// weight shuffle and the all-reduce form, and every op's fake).
TORCH_LIBRARY_FRAGMENT(arn, m) {
  m.def("rmsnorm(Tensor x, Tensor? weight, float eps) -> Tensor");
  m.def("fused_add_rmsnorm(Tensor x, Tensor(a!) residual, Tensor? weight, float eps) -> Tensor");
  m.def("rmsnorm_fp8_static(Tensor x, Tensor? weight, float eps, Tensor scale) -> Tensor");
  m.def("rmsnorm_fp8_dynamic(Tensor x, Tensor? weight, float eps) -> (Tensor, Tensor)");
  m.def("fused_add_rmsnorm_fp8_static(Tensor x, Tensor(a!) residual, Tensor? weight, float eps, "
        "Tensor scale) -> Tensor");
  m.def("fused_add_rmsnorm_fp8_dynamic(Tensor x, Tensor(a!) residual, Tensor? weight, float eps) "
        "-> (Tensor, Tensor)");
  m.def("silu_and_mul(Tensor x) -> Tensor");
  m.def("silu_and_mul_fp8_static(Tensor x, Tensor scale) -> Tensor");
  m.def("silu_and_mul_fp8_dynamic(Tensor x) -> (Tensor, Tensor)");
  m.def("fp8_gemm(Tensor a, Tensor scale_a, Tensor b, Tensor scale_b, ScalarType? out_dtype=None) "
        "-> Tensor");
  m.def("fp8_gemm_preshuffled(Tensor a, Tensor scale_a, Tensor b_shuffled, int n, int k, "
        "Tensor scale_b, ScalarType? out_dtype=None) -> Tensor");
}

TORCH_LIBRARY_IMPL(arn, CUDA, m) {
  m.impl("rmsnorm", &op_rmsnorm);
  m.impl("fused_add_rmsnorm", &op_fused_add_rmsnorm);
  m.impl("rmsnorm_fp8_static", &op_rmsnorm_fp8_static);
  m.impl("rmsnorm_fp8_dynamic", &op_rmsnorm_fp8_dynamic);
  m.impl("fused_add_rmsnorm_fp8_static", &op_fused_add_rmsnorm_fp8_static);
  m.impl("fused_add_rmsnorm_fp8_dynamic", &op_fused_add_rmsnorm_fp8_dynamic);
  m.impl("silu_and_mul", &op_silu_and_mul);
  m.impl("silu_and_mul_fp8_static", &op_silu_and_mul_fp8_static);
  m.impl("silu_and_mul_fp8_dynamic", &op_silu_and_mul_fp8_dynamic);
  m.impl("fp8_gemm", &op_fp8_gemm);
  m.impl("fp8_gemm_preshuffled", &op_fp8_gemm_preshuffled);
}

PYBIND11_MODULE(_native, m) {
  m.doc() = "argument marshalling of the residual_add_rmsnorm_amd binding (C ABI of libarn.so)";
  m.def("bind", &bind);
  m.def("row_view", &py_row_view);
  m.def("rmsnorm", [](const at::Tensor& x, const OptT& w, double eps, const OptT& out) {
    return from_python([&] { return rmsnorm(x, w, eps, out); });
  });
  m.def("fused_add_rmsnorm",
        [](const at::Tensor& x, const at::Tensor& res, const OptT& w, double eps, const OptT& out) {
          return from_python([&] { return fused_add_rmsnorm(x, res, w, eps, out); });
        });
  m.def("rmsnorm_fp8", [](const at::Tensor& x, const OptT& w, double eps, const OptT& scale,
                          bool dynamic, const OptT& out, const OptT& scales_out) {
    return from_python([&] { return rmsnorm_fp8(x, w, eps, scale, dynamic, out, scales_out); });
  });
  m.def("fused_add_rmsnorm_fp8",
        [](const at::Tensor& x, const at::Tensor& res, const OptT& w, double eps, const OptT& scale,
           bool dynamic, const OptT& out, const OptT& scales_out) {
          return from_python(
              [&] { return fused_add_rmsnorm_fp8(x, res, w, eps, scale, dynamic, out, scales_out); });
        });
  // Returns out, or (codes, scale tensor) for an e4m3 output.
  m.def("norm", [](const at::Tensor& x, const OptT& w, double eps, const OptT& res,
                   int64_t variance_size, const std::string& fp8, const OptT& scale,
                   const OptT& out, const OptT& scales_out) -> py::object {
    const Pair r = from_python(
        [&] { return norm(x, w, eps, res, variance_size, fp8, scale, out, scales_out); });
    if (fp8.empty()) return py::cast(std::get<0>(r));
    return py::cast(r);
  });
  m.def("silu_and_mul", [](const at::Tensor& x, const OptT& out) {
    return from_python([&] { return silu_and_mul(x, out); });
  });
  m.def("silu_and_mul_fp8", [](const at::Tensor& x, const OptT& scale, bool dynamic,
                               const OptT& out, const OptT& scales_out) {
    return from_python([&] { return silu_and_mul_fp8(x, scale, dynamic, out, scales_out); });
  });
  m.def("fp8_gemm", [](const at::Tensor& a, const at::Tensor& sa, const at::Tensor& b,
                       const at::Tensor& sb, int out_code, const OptT& out, const OptT& ws,
                       int64_t pre_n, int64_t pre_k) {
    return from_python([&] { return fp8_gemm(a, sa, b, sb, out_code, out, ws, pre_n, pre_k); });
  });
  m.def("fp8_gemm_preshuffled_noalloc",
        [](const at::Tensor& a, const at::Tensor& sa, const at::Tensor& b, int64_t n, int64_t kb,
           const at::Tensor& sb, int out_code, const OptT& out) {
          return from_python(
              [&] { return fp8_gemm_preshuffled_noalloc(a, sa, b, n, kb, sb, out_code, out); });
        });
}
