// C ABI of h3dit: argument validation, workspace carving and the launch
// sequence of the DiT block.  Every check runs on the host before anything is
// enqueued; a failed check returns a status and launches nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/h3dit.h"
#include "h3_common.hpp"
#include "h3_kernels.hpp"

namespace {

thread_local char g_err[512] = "";

h3_status fail(h3_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

h3_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return H3_OK;
  return fail(H3_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t esize(h3_dtype dt) { return dt == H3_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define CHECK(cond, ...)                              \
  do {                                                \
    if (!(cond)) return fail(H3_ERR_ARG, __VA_ARGS__); \
  } while (0)

h3_status check_dtype(h3_dtype dt) {
  if (dt != H3_F32 && dt != H3_BF16) return fail(H3_ERR_UNSUPPORTED, "dtype %d not supported", (int)dt);
  return H3_OK;
}

// tensor pointer p of rows with stride ld (elements) and width w (elements)
h3_status check_rows(const char* name, const void* p, int64_t ld, int64_t width, int64_t rows,
                     h3_dtype dt, bool required = true) {
  if (!p) {
    if (required && rows > 0) return fail(H3_ERR_ARG, "%s is NULL", name);
    return H3_OK;
  }
  if (!aligned16(p)) return fail(H3_ERR_ARG, "%s is not 16-byte aligned", name);
  if (ld < 0 || (ld != 0 && ld < width))
    return fail(H3_ERR_ARG, "%s: row stride %lld below row width %lld", name, (long long)ld,
                (long long)width);
  if ((ld * (int64_t)esize(dt)) % 16 != 0)
    return fail(H3_ERR_ARG, "%s: row stride %lld elements is not a multiple of 16 bytes", name,
                (long long)ld);
  return H3_OK;
}

// Device check, cached per device: gfx950 only.
std::atomic<int> g_dev_ok[64];

h3_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(H3_ERR_UNSUPPORTED, "device ordinal %d", dev);
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(H3_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return H3_OK;
}

#define TRY(expr)                          \
  do {                                     \
    h3_status _st = (expr);                \
    if (_st != H3_OK) return _st;          \
  } while (0)

h3_status check_head_dim(int32_t d) {
  if (d != 64 && d != 128) return fail(H3_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d);
  return H3_OK;
}

h3_status check_sections(int32_t d, int32_t st, int32_t sh, int32_t sw) {
  CHECK(st >= 0 && sh >= 0 && sw >= 0, "negative RoPE section");
  CHECK(st % 2 == 0 && sh % 2 == 0 && sw % 2 == 0, "RoPE sections must be even (%d,%d,%d)", st, sh, sw);
  CHECK(st + sh + sw == d, "RoPE sections %d+%d+%d do not sum to head_dim %d", st, sh, sw, d);
  return H3_OK;
}

h3_status validate_qk(void* q, int64_t ld_q, void* k, int64_t ld_k, int64_t n_tok, int32_t H,
                      int32_t D, const void* g_q, const void* g_k, const h3_pos* pos,
                      int32_t st, int32_t sh, int32_t sw, float theta, float eps, h3_dtype dt) {
  TRY(check_dtype(dt));
  CHECK(n_tok >= 0, "n_tok < 0");
  CHECK(H > 0, "n_heads must be positive");
  TRY(check_head_dim(D));
  TRY(check_sections(D, st, sh, sw));
  CHECK(theta > 0.f && std::isfinite(theta), "theta must be positive");
  CHECK(eps >= 0.f, "eps < 0");
  if (n_tok == 0) return H3_OK;
  TRY(check_rows("q", q, ld_q, (int64_t)H * D, n_tok, dt));
  TRY(check_rows("k", k, ld_k, (int64_t)H * D, n_tok, dt));
  CHECK(ld_q > 0 && ld_k > 0, "q/k row stride must be positive");
  CHECK(g_q && g_k, "gains are NULL");
  CHECK(aligned16(g_q) && aligned16(g_k), "gains are not 16-byte aligned");
  CHECK(pos && aligned16(pos), "pos is NULL or not 16-byte aligned");
  return H3_OK;
}

h3_status validate_attn(const void* q, int64_t ld_q, const void* k, int64_t ld_k, const void* v,
                        int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf, int32_t H,
                        int32_t D, const int32_t* cu, int32_t n_seg, int32_t max_len,
                        void* ws, size_t ws_bytes, h3_dtype dt, bool fp8 = false,
                        bool ws_from_library = false) {
  TRY(check_dtype(dt));
  CHECK(n_buf >= 0 && n_buf < (int64_t)INT32_MAX, "n_buf out of range");
  CHECK(H > 0, "n_heads must be positive");
  TRY(check_head_dim(D));
  CHECK(n_seg >= 1 && n_seg <= 65535, "n_seg must be in [1, 65535]");
  CHECK(max_len >= 0 && max_len <= n_buf, "max_valid_len must be in [0, n_buf]");
  CHECK(cu != nullptr, "cu_slots is NULL");
  if (n_buf == 0) return H3_OK;
  const int64_t w = (int64_t)H * D;
  TRY(check_rows("q", q, ld_q, w, n_buf, dt));
  TRY(check_rows("k", k, ld_k, w, n_buf, dt));
  TRY(check_rows("v", v, ld_v, w, n_buf, dt));
  TRY(check_rows("o", o, ld_o, w, n_buf, dt));
  CHECK(ld_q > 0 && ld_k > 0 && ld_v > 0 && ld_o > 0, "row strides must be positive");
  // the bf16 kernel addresses a 64-row key tile and the transposed-V scratch with 32-bit byte offsets
  CHECK(ld_k <= (1 << 23) && n_buf <= (1 << 22), "row stride above 2^23 or n_buf above 2^22");
  // ... and a head's transposed V (D rows of vt_columns keys, 2 bytes each) likewise
  CHECK((int64_t)D * h3::vt_columns(n_buf, n_seg) * 2 <= (int64_t)INT32_MAX,
        "n_buf %lld with %d segments: a head's transposed V exceeds 2^31 bytes", (long long)n_buf, n_seg);
  if (ws_from_library) return H3_OK;
  const size_t need = fp8 ? h3::attn_fp8_workspace_bytes(n_buf, H, D, n_seg)
                         : h3::attn_workspace_bytes(dt == H3_BF16, n_buf, H, D, n_seg);
  if (ws_bytes < need)
    return fail(H3_ERR_WORKSPACE, "attention workspace %zu bytes, need %zu", ws_bytes, need);
  CHECK(need == 0 || (ws && aligned16(ws)), "workspace is NULL or not 16-byte aligned");
  return H3_OK;
}

// Segment metadata in host memory: 0 <= cu[0] <= ... <= cu[n_seg] <= n_buf, and every valid
// length (the slot length where valid is NULL) in [0, slot length] and at most max_len.
h3_status check_segments_host(const int32_t* cu, const int32_t* valid, int32_t n_seg,
                              int64_t n_buf, int32_t max_len) {
  CHECK(cu, "cu_slots is NULL");
  CHECK(n_seg >= 1 && n_seg <= 65535, "n_seg must be in [1, 65535]");
  CHECK(n_buf >= 0 && n_buf < (int64_t)INT32_MAX, "n_buf out of range");
  CHECK(cu[0] >= 0, "cu_slots[0] = %d is negative", cu[0]);
  for (int32_t i = 0; i < n_seg; ++i)
    CHECK(cu[i + 1] >= cu[i], "cu_slots decreases at %d (%d -> %d)", i, cu[i], cu[i + 1]);
  CHECK((int64_t)cu[n_seg] <= n_buf, "cu_slots[n_seg] = %d exceeds n_buf = %lld", cu[n_seg],
        (long long)n_buf);
  for (int32_t i = 0; i < n_seg; ++i) {
    const int32_t slot = cu[i + 1] - cu[i];
    const int32_t len = valid ? valid[i] : slot;
    CHECK(len >= 0 && len <= slot, "valid_len[%d] = %d outside [0, %d]", i, len, slot);
    CHECK(len <= max_len, "valid length %d of segment %d exceeds max_valid_len = %d", len, i,
          max_len);
  }
  return H3_OK;
}

// H3_DEBUG_VALIDATE=1: copy the device segment metadata to the host (this synchronises the
// stream) and check it before anything is launched.
h3_status debug_check_segments(const int32_t* cu_dev, const int32_t* valid_dev, int32_t n_seg,
                               int64_t n_buf, int32_t max_len, hipStream_t s) {
  const char* e = getenv("H3_DEBUG_VALIDATE");
  if (!e || strcmp(e, "1") != 0) return H3_OK;
  std::vector<int32_t> cu((size_t)n_seg + 1), vl(valid_dev ? (size_t)n_seg : 0);
  TRY(hip_status(hipMemcpyAsync(cu.data(), cu_dev, cu.size() * 4, hipMemcpyDeviceToHost, s),
                 "H3_DEBUG_VALIDATE copy of cu_slots"));
  if (valid_dev)
    TRY(hip_status(hipMemcpyAsync(vl.data(), valid_dev, vl.size() * 4, hipMemcpyDeviceToHost, s),
                   "H3_DEBUG_VALIDATE copy of valid_len"));
  TRY(hip_status(hipStreamSynchronize(s), "H3_DEBUG_VALIDATE synchronisation"));
  return check_segments_host(cu.data(), valid_dev ? vl.data() : nullptr, n_seg, n_buf, max_len);
}

h3_status validate_modres(void* x, int64_t ld_x, const void* y, int64_t ld_y, const void* gate,
                          const void* shift, const void* scale, int64_t ld_mod, void* h,
                          int64_t ld_h, int64_t n_tok, int32_t dim, int32_t norm_kind, float eps,
                          h3_dtype dt) {
  TRY(check_dtype(dt));
  CHECK(n_tok >= 0 && n_tok <= (int64_t)INT32_MAX, "n_tok out of range");
  CHECK(dim > 0 && dim % 8 == 0 && dim <= 16384, "dim must be a positive multiple of 8, <= 16384");
  CHECK(norm_kind == 0 || norm_kind == 1, "norm_kind must be 0 or 1");
  CHECK(eps >= 0.f, "eps < 0");
  if (n_tok == 0) return H3_OK;
  TRY(check_rows("x", x, ld_x, dim, n_tok, dt));
  CHECK(ld_x > 0, "x row stride must be positive");
  CHECK(y || h, "nothing to do: y and h_out are both NULL");
  if (y) {
    TRY(check_rows("y", y, ld_y, dim, n_tok, dt));
    CHECK(ld_y > 0, "y row stride must be positive");
    TRY(check_rows("gate", gate, ld_mod, dim, n_tok, dt));
  }
  if (h) {
    TRY(check_rows("h_out", h, ld_h, dim, n_tok, dt));
    CHECK(ld_h > 0, "h_out row stride must be positive");
    TRY(check_rows("shift", shift, ld_mod, dim, n_tok, dt));
    TRY(check_rows("scale", scale, ld_mod, dim, n_tok, dt));
  }
  return H3_OK;
}

h3_status validate_linear(const void* a, int64_t lda, const void* w, int64_t ldw, void* out,
                          int64_t ld_out, int64_t m, int32_t n_out, int32_t k_in,
                          const void* gate, int64_t ld_gate, h3_dtype dt) {
  TRY(check_dtype(dt));
  CHECK(m >= 0 && m <= (int64_t)INT32_MAX, "m out of range");
  CHECK(n_out > 0 && k_in > 0 && k_in % 8 == 0, "n_out > 0 and k_in a positive multiple of 8 required");
  if (m == 0) return H3_OK;
  TRY(check_rows("a", a, lda, k_in, m, dt));
  TRY(check_rows("w", w, ldw, k_in, n_out, dt));
  TRY(check_rows("out", out, ld_out, n_out, m, dt));
  CHECK(lda > 0 && ldw > 0 && ld_out > 0, "row strides must be positive");
  if (gate) TRY(check_rows("gate", gate, ld_gate, n_out, m, dt));
  return H3_OK;
}

// MX operand of logical width k (columns) with `rows` rows
h3_status check_mx(const char* name, const h3_mx_operand* x, int64_t k, int64_t rows) {
  if (!x) return fail(H3_ERR_ARG, "%s is NULL", name);
  const int64_t kp = h3::round_up(k, 128);
  if (!x->data || !aligned16(x->data)) return fail(H3_ERR_ARG, "%s: data NULL or not 16-byte aligned", name);
  if (x->ld < kp || x->ld % 16 != 0 || x->ld > (1 << 23))
    return fail(H3_ERR_ARG, "%s: ld %lld must be a multiple of 16 in [%lld, 2^23]", name,
                (long long)x->ld, (long long)kp);
  if (!x->scale || ((uintptr_t)x->scale & 3u) != 0)
    return fail(H3_ERR_ARG, "%s: scale NULL or not 4-byte aligned", name);
  if (x->ld_scale < kp / 32 || x->ld_scale % 4 != 0)
    return fail(H3_ERR_ARG, "%s: ld_scale %lld must be a multiple of 4, >= %lld", name,
                (long long)x->ld_scale, (long long)(kp / 32));
  (void)rows;
  return H3_OK;
}

h3::MxOperand mx_of(const h3_mx_operand* x) {
  h3::MxOperand m;
  m.data = x->data;
  m.ld = x->ld;
  m.scale = x->scale;
  m.ld_scale = x->ld_scale;
  return m;
}

// bf16 g (only where a separate pass quantizes it: ffn_dim % 128 != 0), then
// its MX operand
int64_t swiglu_fp8_parts(int64_t n_tok, int32_t ffn_dim, int64_t* g_q, int64_t* g_s) {
  const int64_t fp = h3::round_up(ffn_dim, 128);
  const int64_t g = ffn_dim % 128 == 0 ? 0 : h3::round_up(n_tok * ffn_dim * 2, 256);
  *g_q = g;
  *g_s = g + h3::round_up(n_tok * fp, 256);
  return *g_s + h3::round_up(n_tok * (fp / 32), 256);
}

}  // namespace

// Scratch of h3_varlen_attn_noalloc (the transposed copy of v): one copy per
// device, held until the process ends.  Host code never passes `scratch`
// itself to a kernel: it is a host-side stand-in for the device variable;
// its device address comes from hipGetSymbolAddress, once per device.
static constexpr size_t kNoAllocScratchBytes = (size_t)H3_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::once_flag g_scratch_once[64];
void* g_scratch_ptr[64];
hipError_t g_scratch_err[64];

// device address of `scratch` on the current device (looked up on the first
// call on that device, with the device current)
h3_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(H3_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess)
    return hip_status(g_scratch_err[dev], "hipGetSymbolAddress of the no-allocation scratch");
  if (!g_scratch_ptr[dev] || ((uintptr_t)g_scratch_ptr[dev] & 255u) != 0)
    return fail(H3_ERR_HIP, "no-allocation scratch: bad device address");
  *out = g_scratch_ptr[dev];
  return H3_OK;
}
}  // namespace

using namespace h3;

extern "C" {

int h3_abi_version(void) { return H3_ABI_VERSION; }

const char* h3_status_string(h3_status st) {
  switch (st) {
    case H3_OK: return "ok";
    case H3_ERR_ARG: return "invalid argument";
    case H3_ERR_UNSUPPORTED: return "unsupported";
    case H3_ERR_WORKSPACE: return "workspace too small";
    case H3_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* h3_last_error(void) { return g_err; }

h3_status h3_qk_norm_rope(void* q, int64_t ld_q, void* k, int64_t ld_k, int64_t n_tok,
                          int32_t n_heads, int32_t head_dim, const void* g_q, const void* g_k,
                          const h3_pos* pos, int32_t sec_t, int32_t sec_h, int32_t sec_w,
                          float theta, float eps, h3_dtype dtype, void* stream) {
  g_err[0] = 0;
  TRY(validate_qk(q, ld_q, k, ld_k, n_tok, n_heads, head_dim, g_q, g_k, pos, sec_t, sec_h, sec_w,
                  theta, eps, dtype));
  if (n_tok == 0) return H3_OK;
  TRY(check_device());
  return hip_status(launch_qk_norm_rope(dtype == H3_BF16, head_dim, q, ld_q, k, ld_k, n_tok,
                                        n_heads, g_q, g_k, pos, sec_t, sec_h, theta, eps,
                                        (hipStream_t)stream),
                    "qk_norm_rope launch");
}

h3_status h3_check_segments(const int32_t* cu_slots, const int32_t* valid_len, int32_t n_seg,
                            int64_t n_buf, int32_t max_valid_len) {
  g_err[0] = 0;
  return check_segments_host(cu_slots, valid_len, n_seg, n_buf, max_valid_len);
}

size_t h3_varlen_attn_workspace_size(int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                     int32_t n_seg, h3_dtype dtype) {
  if (n_buf <= 0 || n_heads <= 0 || head_dim <= 0 || n_seg <= 0) return 0;
  return attn_workspace_bytes(dtype == H3_BF16, n_buf, n_heads, head_dim, n_seg);
}

h3_status h3_varlen_attn(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                         const void* v, int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf,
                         int32_t n_heads, int32_t head_dim, const int32_t* cu_slots,
                         const int32_t* valid_len, int32_t n_seg, int32_t max_valid_len,
                         float softmax_scale, void* ws, size_t ws_bytes, h3_dtype dtype,
                         void* stream) {
  g_err[0] = 0;
  TRY(validate_attn(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, head_dim, cu_slots, n_seg,
                    max_valid_len, ws, ws_bytes, dtype));
  if (n_buf == 0) return H3_OK;
  TRY(check_device());
  TRY(debug_check_segments(cu_slots, valid_len, n_seg, n_buf, max_valid_len, (hipStream_t)stream));
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  return hip_status(launch_varlen_attn(dtype == H3_BF16, head_dim, q, ld_q, k, ld_k, v, ld_v, o,
                                       ld_o, n_buf, n_heads, cu_slots, valid_len, n_seg,
                                       max_valid_len, scale, ws, (hipStream_t)stream),
                    "varlen_attn launch");
}

h3_status h3_varlen_attn_noalloc(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                                 const void* v, int64_t ld_v, void* o, int64_t ld_o,
                                 int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                 const int32_t* cu_slots, const int32_t* valid_len,
                                 int32_t n_seg, int32_t max_valid_len, float softmax_scale,
                                 h3_dtype dtype, void* stream) {
  g_err[0] = 0;
  TRY(validate_attn(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, head_dim, cu_slots, n_seg,
                    max_valid_len, nullptr, 0, dtype, false, true));
  if (n_buf == 0) return H3_OK;
  const size_t need = attn_workspace_bytes(dtype == H3_BF16, n_buf, n_heads, head_dim, n_seg);
  if (need > kNoAllocScratchBytes)
    return fail(H3_ERR_WORKSPACE,
                "h3_varlen_attn_noalloc: this call needs %zu bytes of scratch, above the fixed "
                "%zu (n_heads x head_dim x (n_buf + 128 (n_seg + 1)) x 2 bytes); use "
                "h3_varlen_attn with a workspace",
                need, kNoAllocScratchBytes);
  TRY(check_device());
  void* ws = nullptr;
  TRY(scratch_of_current_device(&ws));
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  return hip_status(launch_varlen_attn(dtype == H3_BF16, head_dim, q, ld_q, k, ld_k, v, ld_v, o,
                                       ld_o, n_buf, n_heads, cu_slots, valid_len, n_seg,
                                       max_valid_len, scale, ws, (hipStream_t)stream),
                    "varlen_attn_noalloc launch");
}

h3_status h3_varlen_attn_skip(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                              const void* v, int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf,
                              int32_t n_heads, int32_t head_dim, const int32_t* cu_slots,
                              const int32_t* valid_len, int32_t n_seg, int32_t max_valid_len,
                              float softmax_scale, float skip_log2, void* ws, size_t ws_bytes,
                              h3_dtype dtype, void* stream) {
  g_err[0] = 0;
  if (dtype != H3_BF16) return fail(H3_ERR_UNSUPPORTED, "Skip-Softmax attention takes bf16 operands");
  CHECK(skip_log2 < 0.f, "skip_log2 must be negative (-inf: never skip)");
  TRY(validate_attn(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, head_dim, cu_slots, n_seg,
                    max_valid_len, ws, ws_bytes, dtype));
  if (n_buf == 0) return H3_OK;
  TRY(check_device());
  TRY(debug_check_segments(cu_slots, valid_len, n_seg, n_buf, max_valid_len, (hipStream_t)stream));
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  return hip_status(launch_varlen_attn_skip(head_dim, q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf,
                                            n_heads, cu_slots, valid_len, n_seg, max_valid_len,
                                            scale, skip_log2, ws, (hipStream_t)stream),
                    "varlen_attn_skip launch");
}

size_t h3_varlen_attn_fp8_workspace_size(int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                         int32_t n_seg) {
  if (n_buf <= 0 || n_heads <= 0 || head_dim <= 0 || n_seg <= 0) return 0;
  return attn_fp8_workspace_bytes(n_buf, n_heads, head_dim, n_seg);
}

namespace {
h3_status varlen_attn_fp8(const void* q, int64_t ld_q, const void* k, int64_t ld_k, const void* v,
                          int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf, int32_t n_heads,
                          int32_t head_dim, const int32_t* cu_slots, const int32_t* valid_len,
                          int32_t n_seg, int32_t max_valid_len, float softmax_scale,
                          float skip_log2, void* ws, size_t ws_bytes, h3_dtype dtype,
                          void* stream) {
  if (dtype != H3_BF16) return fail(H3_ERR_UNSUPPORTED, "the FP8 attention takes bf16 operands");
  TRY(validate_attn(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, head_dim, cu_slots, n_seg,
                    max_valid_len, ws, ws_bytes, dtype, true));
  if (n_buf == 0) return H3_OK;
  TRY(check_device());
  TRY(debug_check_segments(cu_slots, valid_len, n_seg, n_buf, max_valid_len, (hipStream_t)stream));
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  return hip_status(launch_varlen_attn_fp8(head_dim, q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf,
                                           n_heads, cu_slots, valid_len, n_seg, max_valid_len,
                                           scale, skip_log2, ws, (hipStream_t)stream),
                    "varlen_attn_fp8 launch");
}
}  // namespace

h3_status h3_varlen_attn_fp8(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                             const void* v, int64_t ld_v, void* o, int64_t ld_o, int64_t n_buf,
                             int32_t n_heads, int32_t head_dim, const int32_t* cu_slots,
                             const int32_t* valid_len, int32_t n_seg, int32_t max_valid_len,
                             float softmax_scale, void* ws, size_t ws_bytes, h3_dtype dtype,
                             void* stream) {
  g_err[0] = 0;
  return varlen_attn_fp8(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, head_dim, cu_slots,
                         valid_len, n_seg, max_valid_len, softmax_scale, 0.f, ws, ws_bytes, dtype,
                         stream);
}

h3_status h3_varlen_attn_fp8_skip(const void* q, int64_t ld_q, const void* k, int64_t ld_k,
                                  const void* v, int64_t ld_v, void* o, int64_t ld_o,
                                  int64_t n_buf, int32_t n_heads, int32_t head_dim,
                                  const int32_t* cu_slots, const int32_t* valid_len,
                                  int32_t n_seg, int32_t max_valid_len, float softmax_scale,
                                  float skip_log2, void* ws, size_t ws_bytes, h3_dtype dtype,
                                  void* stream) {
  g_err[0] = 0;
  CHECK(skip_log2 < 0.f, "skip_log2 must be negative (-inf: never skip)");
  return varlen_attn_fp8(q, ld_q, k, ld_k, v, ld_v, o, ld_o, n_buf, n_heads, head_dim, cu_slots,
                         valid_len, n_seg, max_valid_len, softmax_scale, skip_log2, ws, ws_bytes,
                         dtype, stream);
}

h3_status h3_modulate_residual(void* x, int64_t ld_x, const void* y, int64_t ld_y,
                               const void* gate, const void* shift, const void* scale,
                               int64_t ld_mod, void* h_out, int64_t ld_h, int64_t n_tok,
                               int32_t dim, int32_t norm_kind, float eps, h3_dtype dtype,
                               void* stream) {
  g_err[0] = 0;
  TRY(validate_modres(x, ld_x, y, ld_y, gate, shift, scale, ld_mod, h_out, ld_h, n_tok, dim,
                      norm_kind, eps, dtype));
  if (n_tok == 0) return H3_OK;
  TRY(check_device());
  return hip_status(launch_modulate_residual(dtype == H3_BF16, x, ld_x, y, ld_y, gate, shift,
                                             scale, ld_mod, h_out, ld_h, n_tok, dim, norm_kind,
                                             eps, (hipStream_t)stream),
                    "modulate_residual launch");
}

h3_status h3_linear(const void* a, int64_t lda, const void* w, int64_t ldw, void* out,
                    int64_t ld_out, int64_t m, int32_t n_out, int32_t k_in, const void* gate,
                    int64_t ld_gate, h3_dtype dtype, void* stream) {
  g_err[0] = 0;
  TRY(validate_linear(a, lda, w, ldw, out, ld_out, m, n_out, k_in, gate, ld_gate, dtype));
  if (m == 0) return H3_OK;
  TRY(check_device());
  return hip_status(launch_gemm(dtype == H3_BF16, gate ? EPI_RESIDUAL : EPI_STORE, a, lda, w,
                                nullptr, ldw, out, ld_out, gate, ld_gate, m, n_out, k_in,
                                (hipStream_t)stream),
                    "linear launch");
}

size_t h3_swiglu_workspace_size(int64_t n_tok, int32_t ffn_dim, h3_dtype dtype) {
  if (n_tok <= 0 || ffn_dim <= 0) return 0;
  return (size_t)round_up((int64_t)n_tok * ffn_dim * (int64_t)esize(dtype), 256);
}

h3_status h3_swiglu(const void* h, int64_t ld_h, const void* w1, const void* w3,
                    const void* w2, void* out, int64_t ld_out, const void* gate,
                    int64_t ld_gate, int64_t n_tok, int32_t dim, int32_t ffn_dim, void* ws,
                    size_t ws_bytes, h3_dtype dtype, void* stream) {
  g_err[0] = 0;
  TRY(check_dtype(dtype));
  CHECK(n_tok >= 0 && n_tok <= (int64_t)INT32_MAX, "n_tok out of range");
  CHECK(dim > 0 && dim % 8 == 0 && ffn_dim > 0 && ffn_dim % 8 == 0,
        "dim and ffn_dim must be positive multiples of 8");
  if (n_tok == 0) return H3_OK;
  TRY(check_rows("h", h, ld_h, dim, n_tok, dtype));
  TRY(check_rows("w1", w1, dim, dim, ffn_dim, dtype));
  TRY(check_rows("w3", w3, dim, dim, ffn_dim, dtype));
  TRY(check_rows("w2", w2, ffn_dim, ffn_dim, dim, dtype));
  TRY(check_rows("out", out, ld_out, dim, n_tok, dtype));
  CHECK(ld_h > 0 && ld_out > 0, "row strides must be positive");
  if (gate) TRY(check_rows("gate", gate, ld_gate, dim, n_tok, dtype));
  const size_t need = h3_swiglu_workspace_size(n_tok, ffn_dim, dtype);
  if (ws_bytes < need) return fail(H3_ERR_WORKSPACE, "swiglu workspace %zu bytes, need %zu", ws_bytes, need);
  CHECK(ws && aligned16(ws), "workspace is NULL or not 16-byte aligned");
  TRY(check_device());
  const bool bf = dtype == H3_BF16;
  hipStream_t s = (hipStream_t)stream;
  TRY(hip_status(launch_gemm(bf, EPI_SWIGLU, h, ld_h, w1, w3, dim, ws, ffn_dim, nullptr, 0, n_tok,
                             ffn_dim, dim, s),
                 "swiglu up-projection launch"));
  return hip_status(launch_gemm(bf, gate ? EPI_RESIDUAL : EPI_STORE, ws, ffn_dim, w2, nullptr,
                                ffn_dim, out, ld_out, gate, ld_gate, n_tok, dim, ffn_dim, s),
                    "swiglu down-projection launch");
}

// ------------------------------------------------ FP8 (MX e4m3) projections

h3_status h3_mx_quantize(const void* x, int64_t ld_x, int64_t rows, int32_t cols, void* q,
                         int64_t ld_q, void* scale, int64_t ld_scale, h3_dtype dtype,
                         void* stream) {
  g_err[0] = 0;
  if (dtype != H3_BF16) return fail(H3_ERR_UNSUPPORTED, "MX quantization takes bf16 input");
  CHECK(rows >= 0 && rows <= (int64_t)INT32_MAX * 4, "rows out of range");
  CHECK(cols > 0 && cols % 32 == 0, "cols must be a positive multiple of 32");
  if (rows == 0) return H3_OK;
  TRY(check_rows("x", x, ld_x, cols, rows, H3_BF16));
  CHECK(ld_x > 0, "x row stride must be positive");
  h3_mx_operand o{q, ld_q, scale, ld_scale};
  TRY(check_mx("q", &o, cols, rows));
  TRY(check_device());
  return hip_status(launch_mx_quantize(x, ld_x, rows, cols, q, ld_q, scale, ld_scale,
                                       (hipStream_t)stream),
                    "mx_quantize launch");
}

h3_status h3_modulate_mx(const void* x, int64_t ld_x, const void* shift, const void* scale,
                         int64_t ld_mod, void* q, int64_t ld_q, void* q_scale, int64_t ld_scale,
                         int64_t n_tok, int32_t dim, int32_t norm_kind, float eps, void* stream) {
  g_err[0] = 0;
  CHECK(n_tok >= 0 && n_tok <= (int64_t)INT32_MAX, "n_tok out of range");
  CHECK(dim > 0 && dim % 128 == 0 && dim <= 16384, "dim must be a positive multiple of 128, <= 16384");
  CHECK(norm_kind == 0 || norm_kind == 1, "norm_kind must be 0 or 1");
  CHECK(eps >= 0.f, "eps < 0");
  if (n_tok == 0) return H3_OK;
  TRY(check_rows("x", x, ld_x, dim, n_tok, H3_BF16));
  CHECK(ld_x > 0, "x row stride must be positive");
  TRY(check_rows("shift", shift, ld_mod, dim, n_tok, H3_BF16));
  TRY(check_rows("scale", scale, ld_mod, dim, n_tok, H3_BF16));
  h3_mx_operand o{q, ld_q, q_scale, ld_scale};
  TRY(check_mx("q", &o, dim, n_tok));
  TRY(check_device());
  return hip_status(launch_modulate_mx(x, ld_x, shift, scale, ld_mod, q, ld_q, q_scale, ld_scale,
                                       n_tok, dim, norm_kind, eps, (hipStream_t)stream),
                    "modulate_mx launch");
}

h3_status h3_linear_fp8(const h3_mx_operand* a, const h3_mx_operand* w, void* out,
                        int64_t ld_out, int64_t m, int32_t n_out, int32_t k_in,
                        const void* gate, int64_t ld_gate, void* stream) {
  g_err[0] = 0;
  CHECK(m >= 0 && m <= (int64_t)INT32_MAX, "m out of range");
  CHECK(n_out > 0 && k_in > 0 && k_in % 32 == 0, "n_out > 0 and k_in a positive multiple of 32 required");
  if (m == 0) return H3_OK;
  TRY(check_mx("a", a, k_in, m));
  TRY(check_mx("w", w, k_in, n_out));
  TRY(check_rows("out", out, ld_out, n_out, m, H3_BF16));
  CHECK(ld_out > 0, "out row stride must be positive");
  if (gate) TRY(check_rows("gate", gate, ld_gate, n_out, m, H3_BF16));
  TRY(check_device());
  return hip_status(launch_gemm_mx8(gate ? EPI_RESIDUAL : EPI_STORE, mx_of(a), mx_of(w), MxOperand{},
                                    out, ld_out, gate, ld_gate, m, n_out, k_in,
                                    (hipStream_t)stream),
                    "linear_fp8 launch");
}

size_t h3_swiglu_fp8_workspace_size(int64_t n_tok, int32_t ffn_dim) {
  if (n_tok <= 0 || ffn_dim <= 0) return 0;
  int64_t gq, gs;
  return (size_t)swiglu_fp8_parts(n_tok, ffn_dim, &gq, &gs);
}

h3_status h3_swiglu_fp8(const h3_mx_operand* h, const h3_mx_operand* w1,
                        const h3_mx_operand* w3, const h3_mx_operand* w2, void* out,
                        int64_t ld_out, const void* gate, int64_t ld_gate, int64_t n_tok,
                        int32_t dim, int32_t ffn_dim, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(n_tok >= 0 && n_tok <= (int64_t)INT32_MAX, "n_tok out of range");
  CHECK(dim > 0 && dim % 32 == 0 && ffn_dim > 0 && ffn_dim % 32 == 0,
        "dim and ffn_dim must be positive multiples of 32");
  if (n_tok == 0) return H3_OK;
  TRY(check_mx("h", h, dim, n_tok));
  TRY(check_mx("w1", w1, dim, ffn_dim));
  TRY(check_mx("w3", w3, dim, ffn_dim));
  CHECK(w1->ld == w3->ld && w1->ld_scale == w3->ld_scale, "w1 and w3 must share ld and ld_scale");
  TRY(check_mx("w2", w2, ffn_dim, dim));
  TRY(check_rows("out", out, ld_out, dim, n_tok, H3_BF16));
  CHECK(ld_out > 0, "out row stride must be positive");
  if (gate) TRY(check_rows("gate", gate, ld_gate, dim, n_tok, H3_BF16));
  int64_t gq_off, gs_off;
  const size_t need = (size_t)swiglu_fp8_parts(n_tok, ffn_dim, &gq_off, &gs_off);
  if (ws_bytes < need) return fail(H3_ERR_WORKSPACE, "swiglu_fp8 workspace %zu bytes, need %zu", ws_bytes, need);
  CHECK(ws && aligned16(ws), "workspace is NULL or not 16-byte aligned");
  TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const int64_t fp = round_up(ffn_dim, 128);
  MxOperand g8;
  g8.data = wsb + gq_off;
  g8.ld = fp;
  g8.scale = wsb + gs_off;
  g8.ld_scale = fp / 32;
  // with ffn_dim % 128 == 0 the up-projection's epilogue writes g only as its
  // MX operand (no padding columns); otherwise g is stored in bf16 and a
  // separate pass quantizes it
  GemmMap gmx;
  if (ffn_dim % 128 == 0) {
    gmx.mx_q = (uint8_t*)(wsb + gq_off);
    gmx.mx_ld = fp;
    gmx.mx_s = (uint8_t*)(wsb + gs_off);
    gmx.mx_lds = fp / 32;
    gmx.mx_only = true;
  }
  TRY(hip_status(launch_gemm_mx8(EPI_SWIGLU, mx_of(h), mx_of(w1), mx_of(w3), wsb, ffn_dim,
                                 nullptr, 0, n_tok, ffn_dim, dim, s, gmx),
                 "swiglu_fp8 up-projection launch"));
  if (!gmx.mx_q)
    TRY(hip_status(launch_mx_quantize(wsb, ffn_dim, n_tok, ffn_dim, wsb + gq_off, fp,
                                      wsb + gs_off, fp / 32, s),
                   "swiglu_fp8 gate quantization launch"));
  return hip_status(launch_gemm_mx8(gate ? EPI_RESIDUAL : EPI_STORE, g8, mx_of(w2), MxOperand{},
                                    out, ld_out, gate, ld_gate, n_tok, dim, ffn_dim, s),
                    "swiglu_fp8 down-projection launch");
}

// ------------------------------------------------------------------- block

namespace {
struct BlockWs {
  size_t h1, qkv, attn, o, g, xq, xs, gq, gs, total;
  int64_t xkp, fkp;  // padded widths of the activation and g MX operands
};

// FP8 projections with dim % 128 == 0: the modulated norms write h1 / h2 as
// the MX operand directly (no bf16 h)
bool block_mx_norm(const h3_block_config* c) { return c->gemm_fp8 && c->dim % 128 == 0; }
// FP8 projections with ffn_dim % 128 == 0: the up-projection's epilogue writes
// g only as the MX operand the down-projection reads (no bf16 g)
bool block_g_mx_only(const h3_block_config* c) { return c->gemm_fp8 && c->ffn_dim % 128 == 0; }

// Two groups by lifetime: h1 and the MX activation copy are live across the
// whole block; qkv, the attention workspace and o (world 1) are dead once the
// output projection has read o, before g and its MX copy are first written,
// so the second group starts where the first does.
BlockWs block_ws_layout(const h3_block_config* c, int64_t n, int64_t n_buf, int32_t n_seg,
                        bool share, int32_t head_count) {
  const int64_t es = (int64_t)esize(c->dtype);
  const int64_t hd = (int64_t)c->n_heads * c->head_dim;
  BlockWs w{};
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t at = off;
    off += (size_t)round_up(bytes, 256);
    return at;
  };
  w.h1 = take(block_mx_norm(c) ? 0 : n * c->dim * es);
  if (c->gemm_fp8) {
    // MX copies of the projection inputs: h1 / o / h2 share one (width max(C, H*D)), g its own
    w.xkp = round_up(c->dim > hd ? c->dim : hd, 128);
    w.fkp = round_up(c->ffn_dim, 128);
    w.xq = take(n * w.xkp);
    w.xs = take(n * (w.xkp / 32));
  }
  const size_t stage = off;
  w.qkv = take(n * 3 * hd * es);
  const int64_t an = share ? n_buf : n;
  const int ah = share ? head_count : c->n_heads;
  w.attn = take(c->attn_fp8 ? (int64_t)attn_fp8_workspace_bytes(an, ah, c->head_dim, n_seg)
                            : (int64_t)attn_workspace_bytes(c->dtype == H3_BF16, an, ah,
                                                            c->head_dim, n_seg));
  w.o = take(share ? 0 : n * hd * es);
  const size_t attn_end = off;
  off = stage;
  w.g = take(block_g_mx_only(c) ? 0 : n * (int64_t)c->ffn_dim * es);
  if (c->gemm_fp8) {
    w.gq = take(n * w.fkp);
    w.gs = take(n * (w.fkp / 32));
  }
  w.total = off > attn_end ? off : attn_end;
  return w;
}
}  // namespace

size_t h3_dit_block_workspace_size(const h3_block_config* cfg, int64_t n_tok_local,
                                   int64_t n_buf, int32_t n_seg, int32_t head_count) {
  if (!cfg || n_tok_local < 0 || n_buf < 0 || n_seg <= 0 || head_count < 0) return 0;
  if (head_count > 0) return block_ws_layout(cfg, n_tok_local, n_buf, n_seg, true, head_count).total;
  // 0: cover world 1 and a rank share of any head count
  const size_t w1 = block_ws_layout(cfg, n_tok_local, n_tok_local, n_seg, false, cfg->n_heads).total;
  const size_t sh = block_ws_layout(cfg, n_tok_local, n_buf, n_seg, true, cfg->n_heads).total;
  return w1 > sh ? w1 : sh;
}

h3_status h3_dit_block_forward(const h3_block_config* cfg, const h3_block_weights* w,
                               const h3_block_io* io, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  CHECK(cfg && w && io, "cfg, weights and io must be non-NULL");
  const h3_dtype dt = cfg->dtype;
  TRY(check_dtype(dt));
  const int32_t C = cfg->dim, H = cfg->n_heads, D = cfg->head_dim, F = cfg->ffn_dim;
  CHECK(C > 0 && C % 8 == 0 && C <= 16384, "dim must be a positive multiple of 8, <= 16384");
  CHECK(H > 0 && F > 0 && F % 8 == 0, "n_heads > 0 and ffn_dim a positive multiple of 8 required");
  TRY(check_head_dim(D));
  // they are GEMM widths and row strides of the block's buffers
  CHECK(F <= (1 << 22) && (int64_t)H * D <= (1 << 22), "ffn_dim and n_heads*head_dim must be <= 2^22");
  TRY(check_sections(D, cfg->sec_t, cfg->sec_h, cfg->sec_w));
  CHECK(cfg->norm_kind == 0 || cfg->norm_kind == 1, "norm_kind must be 0 or 1");
  CHECK(cfg->theta > 0.f && cfg->eps_qk >= 0.f && cfg->eps_mod >= 0.f, "theta/eps out of range");
  CHECK(cfg->attn_fp8 == 0 || cfg->attn_fp8 == 1, "attn_fp8 must be 0 or 1");
  CHECK(!cfg->attn_fp8 || dt == H3_BF16, "the FP8 attention path needs bf16 storage");
  CHECK(cfg->gemm_fp8 == 0 || cfg->gemm_fp8 == 1, "gemm_fp8 must be 0 or 1");
  CHECK(cfg->attn_skip_log2 <= 0.f, "attn_skip_log2 must be 0 (off) or negative");
  const bool skip = cfg->attn_skip_log2 < 0.f;
  CHECK(!skip || dt == H3_BF16, "Skip-Softmax attention needs bf16 storage");
  const bool f8 = cfg->gemm_fp8 == 1;
  if (f8) {
    CHECK(dt == H3_BF16, "the FP8 projections need bf16 storage");
    CHECK(C % 32 == 0 && F % 32 == 0 && ((int64_t)H * D) % 32 == 0,
          "the FP8 projections need dim, ffn_dim and n_heads*head_dim multiples of 32");
  }
  const int64_t n = io->n_tok_local;
  CHECK(n >= 0 && n <= (int64_t)INT32_MAX, "n_tok_local out of range");
  const bool share = io->qkv_attn != nullptr;
  const int32_t hb = share ? io->head_begin : 0;
  const int32_t hc = share ? io->head_count : H;
  const bool peer = io->qkv_send != nullptr || io->o_recv != nullptr;
  if (share) {
    CHECK(hc > 0 && hb >= 0 && hb + hc <= H, "head slice [%d, %d) outside [0, %d)", hb, hb + hc, H);
    CHECK(io->tok_begin >= 0 && io->tok_begin + n <= io->n_buf, "local rows outside the buffer");
    if (peer) {
      CHECK(io->qkv_send && io->o_recv && io->o_attn, "peer-major layout needs qkv_send, o_recv, o_attn");
      CHECK(aligned16(io->qkv_attn) && aligned16(io->o_attn) && aligned16(io->qkv_send) &&
                aligned16(io->o_recv),
            "exchange buffers must be 16-byte aligned");
      CHECK(dt == H3_BF16, "the peer-major layout is bf16 only");
      CHECK(H % hc == 0 && hb % hc == 0, "head_count must divide n_heads and head_begin");
      CHECK(io->tok_begin == (int64_t)(hb / hc) * n, "peer-major layout needs tok_begin == rank * n_tok_local");
      CHECK(C % 64 == 0 && ((int64_t)hc * D) % 64 == 0, "peer-major layout needs dim and head_count*D multiples of 64");
    } else {
      CHECK(io->o_attn && io->o_local, "rank-share mode needs qkv_attn, o_attn and o_local");
      CHECK(aligned16(io->qkv_attn) && aligned16(io->o_attn) && aligned16(io->o_local),
            "exchange buffers must be 16-byte aligned");
    }
  } else {
    CHECK(!peer, "qkv_send/o_recv need rank-share mode (qkv_attn)");
    CHECK(io->tok_begin == 0 && io->n_buf == n && (io->head_count == H || io->head_count == 0) &&
              io->head_begin == 0,
          "world-1 mode needs tok_begin 0, n_buf == n_tok_local, full head range");
  }
  if (n == 0) return H3_OK;
  CHECK(io->n_seg >= 1 && io->n_seg <= 65535, "n_seg must be in [1, 65535]");
  CHECK(io->max_valid_len >= 0 && io->max_valid_len <= io->n_buf, "max_valid_len out of range");
  CHECK(io->cu_slots, "cu_slots is NULL");
  CHECK(io->pos && aligned16(io->pos), "pos is NULL or not 16-byte aligned");
  TRY(check_rows("x", io->x, io->ld_x, C, n, dt));
  CHECK(io->ld_x > 0, "x row stride must be positive");
  TRY(check_rows("mod", io->mod, io->ld_mod, 6 * (int64_t)C, n, dt));
  if (f8) {
    CHECK(w->mx, "gemm_fp8 needs the MX weights (weights.mx)");
    const int64_t hd_ = (int64_t)H * D;
    TRY(check_mx("w_qkv (mx)", &w->mx[0], C, 3 * hd_));
    TRY(check_mx("w_o (mx)", &w->mx[1], hd_, C));
    TRY(check_mx("w1 (mx)", &w->mx[2], C, F));
    TRY(check_mx("w3 (mx)", &w->mx[3], C, F));
    TRY(check_mx("w2 (mx)", &w->mx[4], F, C));
    CHECK(w->mx[2].ld == w->mx[3].ld && w->mx[2].ld_scale == w->mx[3].ld_scale,
          "w1 and w3 (mx) must share ld and ld_scale");
    CHECK(w->g_q && w->g_k && aligned16(w->g_q) && aligned16(w->g_k), "a gain pointer is NULL or misaligned");
  } else {
    const void* wp[] = {w->w_qkv, w->w_o, w->w1, w->w3, w->w2, w->g_q, w->g_k};
    for (const void* p : wp) CHECK(p && aligned16(p), "a weight pointer is NULL or misaligned");
  }
  const BlockWs L = block_ws_layout(cfg, n, io->n_buf, io->n_seg, share, hc);
  if (ws_bytes < L.total)
    return fail(H3_ERR_WORKSPACE, "block workspace %zu bytes, need %zu", ws_bytes, L.total);
  CHECK(ws && aligned16(ws), "workspace is NULL or not 16-byte aligned");
  TRY(check_device());
  TRY(debug_check_segments(io->cu_slots, io->valid_len, io->n_seg, io->n_buf, io->max_valid_len,
                           (hipStream_t)stream));

  const bool bf = dt == H3_BF16;
  const int64_t es = (int64_t)esize(dt);
  const int64_t hd = (int64_t)H * D;
  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  void* h1 = wsb + L.h1;
  char* qkv = wsb + L.qkv;
  void* attn_ws = wsb + L.attn;
  char* mod = (char*)io->mod;
  const int64_t ldm = io->ld_mod;
  auto mslot = [&](int i) { return (const void*)(mod + (int64_t)i * C * es); };

  // FP8 projections with C % 128 == 0: the modulated norms write the MX operand
  // of h1 / h2 directly (the same bytes as storing bf16 h and quantizing it)
  const bool mx_norm = block_mx_norm(cfg);
  // A1 h1 = norm(x)(1 + scale1) + shift1
  if (mx_norm) {
    TRY(hip_status(launch_modulate_mx(io->x, io->ld_x, mslot(0), mslot(1), ldm, wsb + L.xq, L.xkp,
                                      wsb + L.xs, L.xkp / 32, n, C, cfg->norm_kind, cfg->eps_mod,
                                      s),
                   "modulate-1 (mx)"));
  } else {
    TRY(hip_status(launch_modulate_residual(bf, io->x, io->ld_x, nullptr, 0, nullptr, mslot(0),
                                            mslot(1), ldm, h1, C, n, C, cfg->norm_kind,
                                            cfg->eps_mod, s),
                   "modulate-1"));
  }
  const float scale = 1.0f / std::sqrt((float)D);
  auto attention = [&](const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                       int64_t ldv, void* o, int64_t ldo, int64_t rows, int heads) {
    if (cfg->attn_fp8)
      return launch_varlen_attn_fp8(D, q, ldq, k, ldk, v, ldv, o, ldo, rows, heads, io->cu_slots,
                                    io->valid_len, io->n_seg, io->max_valid_len, scale,
                                    skip ? cfg->attn_skip_log2 : 0.f, attn_ws, s);
    if (skip)
      return launch_varlen_attn_skip(D, q, ldq, k, ldk, v, ldv, o, ldo, rows, heads,
                                     io->cu_slots, io->valid_len, io->n_seg, io->max_valid_len,
                                     scale, cfg->attn_skip_log2, attn_ws, s);
    return launch_varlen_attn(bf, D, q, ldq, k, ldk, v, ldv, o, ldo, rows, heads, io->cu_slots,
                              io->valid_len, io->n_seg, io->max_valid_len, scale, attn_ws, s);
  };
  // FP8 projections: the activation is quantized into the workspace, then multiplied
  MxOperand xq;
  xq.data = wsb + L.xq;
  xq.ld = L.xkp;
  xq.scale = wsb + L.xs;
  xq.ld_scale = L.xkp / 32;
  auto quant_act = [&](const void* src, int64_t ld_src, int cols, int kgroup = 0,
                       int64_t gstride = 0) {
    return hip_status(launch_mx_quantize(src, ld_src, n, cols, wsb + L.xq, L.xkp, wsb + L.xs,
                                         L.xkp / 32, s, kgroup, gstride),
                      "activation quantization");
  };
  auto wmx = [&](int i) { return f8 ? mx_of(&w->mx[i]) : MxOperand{}; };
  // A3 in the QKV projection's store epilogue (bf16 K % 64 and MX kernels):
  // Q/K RMSNorm + RoPE of the local rows before q and k leave the work-group
  GemmMap qkv_map;
  const bool fuse_qk = bf && C % 64 == 0 && (D == 64 || D == 128);
  if (fuse_qk) {
    qkv_map.qk_pos = (const int4*)io->pos;
    qkv_map.qk_gq = (const bf16_t*)w->g_q;
    qkv_map.qk_gk = (const bf16_t*)w->g_k;
    qkv_map.qk_H = H;
    qkv_map.qk_D = D;
    qkv_map.qk_eps = cfg->eps_qk;
    qkv_map.qk_tab = make_rope_tab(D, cfg->sec_t, cfg->sec_h, cfg->theta);
  }
  if (peer) {
    // Peer-major exchange layout: every all-to-all block is contiguous.
    const int P = H / hc, r = hb / hc;
    const int64_t sd = (int64_t)hc * D;  // slice width
    char* send = (char*)io->qkv_send;
    const int64_t blk = n * 3 * sd * es;  // bytes of one peer block of qkv_send
    // A2 qkv = h1 w_qkv^T, scattered by its epilogue into [P][n][3][hc][D]
    GemmMap scatter = qkv_map;
    scatter.peer_H = H;
    scatter.peer_hc = hc;
    scatter.peer_D = D;
    if (f8) {
      if (!mx_norm) TRY(quant_act(h1, C, C));
      TRY(hip_status(launch_gemm_mx8(EPI_STORE, xq, wmx(0), MxOperand{}, send, 3 * hd, nullptr, 0,
                                     n, (int)(3 * hd), C, s, scatter),
                     "qkv projection (peer-major, fp8)"));
    } else {
      TRY(hip_status(launch_gemm(bf, EPI_STORE, h1, C, w->w_qkv, nullptr, C, send, 3 * hd,
                                 nullptr, 0, n, (int)(3 * hd), C, s, scatter),
                     "qkv projection (peer-major)"));
    }
    // A3 Q/K RMSNorm + RoPE on the local rows, one launch per peer block
    for (int p = 0; p < P && !fuse_qk; ++p) {
      char* b = send + p * blk;
      TRY(hip_status(launch_qk_norm_rope(bf, D, b, 3 * sd, b + sd * es, 3 * sd, n, hc, w->g_q,
                                         w->g_k, io->pos, cfg->sec_t, cfg->sec_h, cfg->theta,
                                         cfg->eps_qk, s),
                     "qk_norm_rope"));
    }
    // A4 the all-to-all's own block: rows [tok_begin, +n) of the attention buffer
    char* qa = (char*)io->qkv_attn;
    TRY(hip_status(hipMemcpyAsync(qa + io->tok_begin * 3 * sd * es, send + r * blk, blk,
                                  hipMemcpyDeviceToDevice, s),
                   "exchange-in self block"));
    // A5 attention over the whole buffer for the head slice
    TRY(hip_status(attention(qa, 3 * sd, qa + sd * es, 3 * sd, qa + 2 * sd * es, 3 * sd,
                             io->o_attn, sd, io->n_buf, hc),
                   "attention"));
    // A6 the reverse all-to-all's own block: o_attn rows [tok_begin, +n) -> o_recv block r
    const int64_t oblk = n * sd * es;
    TRY(hip_status(hipMemcpyAsync((char*)io->o_recv + r * oblk,
                                  (const char*)io->o_attn + io->tok_begin * sd * es, oblk,
                                  hipMemcpyDeviceToDevice, s),
                   "exchange-out self block"));
    // A7 x <- x + gate1 * (o w_o^T), o read from [P][n][hc*D] as K groups of hc*D
    GemmMap grouped;
    grouped.a_kgroup = (int)sd;
    grouped.a_gstride = n * sd;
    if (f8) {
      TRY(quant_act(io->o_recv, sd, (int)hd, (int)sd, n * sd));
      TRY(hip_status(launch_gemm_mx8(EPI_RESIDUAL, xq, wmx(1), MxOperand{}, io->x, io->ld_x,
                                     mslot(2), ldm, n, C, (int)hd, s),
                     "output projection (peer-major, fp8)"));
    } else {
      TRY(hip_status(launch_gemm(bf, EPI_RESIDUAL, io->o_recv, sd, w->w_o, nullptr, hd, io->x,
                                 io->ld_x, mslot(2), ldm, n, C, (int)hd, s, grouped),
                     "output projection (peer-major)"));
    }
  } else {
  // A2 qkv = h1 w_qkv^T
  if (f8) {
    if (!mx_norm) TRY(quant_act(h1, C, C));
    TRY(hip_status(launch_gemm_mx8(EPI_STORE, xq, wmx(0), MxOperand{}, qkv, 3 * hd, nullptr, 0, n,
                                   (int)(3 * hd), C, s, qkv_map),
                   "qkv projection (fp8)"));
  } else {
    TRY(hip_status(launch_gemm(bf, EPI_STORE, h1, C, w->w_qkv, nullptr, C, qkv, 3 * hd, nullptr,
                               0, n, (int)(3 * hd), C, s, qkv_map),
                   "qkv projection"));
  }
  // A3 Q/K RMSNorm + RoPE on the local rows (a pass of its own where the
  // projection's epilogue does not take it)
  if (!fuse_qk)
    TRY(hip_status(launch_qk_norm_rope(bf, D, qkv, 3 * hd, qkv + hd * es, 3 * hd, n, H, w->g_q,
                                       w->g_k, io->pos, cfg->sec_t, cfg->sec_h, cfg->theta,
                                       cfg->eps_qk, s),
                   "qk_norm_rope"));
  const void* o_for_proj;
  if (!share) {
    // A5 attention straight from the QKV buffer
    void* o = wsb + L.o;
    TRY(hip_status(attention(qkv, 3 * hd, qkv + hd * es, 3 * hd, qkv + 2 * hd * es, 3 * hd, o,
                             hd, n, H),
                   "attention"));
    o_for_proj = o;
  } else {
    const int64_t sd = (int64_t)hc * D;  // slice width
    char* qa = (char*)io->qkv_attn;
    // A4 this rank's q, k, v of heads [hb, hb+hc) into its rows of the attention buffer
    TRY(hip_status(launch_copy_rows(qkv + hb * D * es, 3 * hd * es, hd * es,
                                    qa + io->tok_begin * 3 * sd * es, 3 * sd * es, sd * es, n, 3,
                                    sd * es, s),
                   "exchange-in copy"));
    // A5 attention over the whole buffer for the head slice
    TRY(hip_status(attention(qa, 3 * sd, qa + sd * es, 3 * sd, qa + 2 * sd * es, 3 * sd,
                             io->o_attn, sd, io->n_buf, hc),
                   "attention"));
    // A6 this rank's rows of the output into its head slice of o_local
    TRY(hip_status(launch_copy_rows((char*)io->o_attn + io->tok_begin * sd * es, sd * es, 0,
                                    (char*)io->o_local + hb * D * es, hd * es, 0, n, 1, sd * es,
                                    s),
                   "exchange-out copy"));
    o_for_proj = io->o_local;
  }
  // A7 x <- x + gate1 * (o w_o^T)
  if (f8) {
    TRY(quant_act(o_for_proj, hd, (int)hd));
    TRY(hip_status(launch_gemm_mx8(EPI_RESIDUAL, xq, wmx(1), MxOperand{}, io->x, io->ld_x,
                                   mslot(2), ldm, n, C, (int)hd, s),
                   "output projection (fp8)"));
  } else {
    TRY(hip_status(launch_gemm(bf, EPI_RESIDUAL, o_for_proj, hd, w->w_o, nullptr, hd, io->x,
                               io->ld_x, mslot(2), ldm, n, C, (int)hd, s),
                   "output projection"));
  }
  }
  // A8 h2 = norm(x)(1 + scale2) + shift2   (h2 reuses h1's scratch)
  if (mx_norm) {
    TRY(hip_status(launch_modulate_mx(io->x, io->ld_x, mslot(3), mslot(4), ldm, wsb + L.xq, L.xkp,
                                      wsb + L.xs, L.xkp / 32, n, C, cfg->norm_kind, cfg->eps_mod,
                                      s),
                   "modulate-2 (mx)"));
  } else {
    TRY(hip_status(launch_modulate_residual(bf, io->x, io->ld_x, nullptr, 0, nullptr, mslot(3),
                                            mslot(4), ldm, h1, C, n, C, cfg->norm_kind,
                                            cfg->eps_mod, s),
                   "modulate-2"));
  }
  // A9 g = silu(h2 w1^T) * (h2 w3^T)
  void* g = wsb + L.g;
  if (f8) {
    if (!mx_norm) TRY(quant_act(h1, C, C));
    // g's MX operand comes from the up-projection's epilogue when F % 128 == 0,
    // and then only it is written (the down-projection reads nothing else)
    GemmMap gmx;
    if (block_g_mx_only(cfg)) {
      gmx.mx_q = (uint8_t*)(wsb + L.gq);
      gmx.mx_ld = L.fkp;
      gmx.mx_s = (uint8_t*)(wsb + L.gs);
      gmx.mx_lds = L.fkp / 32;
      gmx.mx_only = true;
    }
    TRY(hip_status(launch_gemm_mx8(EPI_SWIGLU, xq, wmx(2), wmx(3), g, F, nullptr, 0, n, F, C, s,
                                   gmx),
                   "swiglu up-projection (fp8)"));
    // A10 x <- x + gate2 * (g w2^T), g quantized on the fly
    if (!gmx.mx_q)
      TRY(hip_status(launch_mx_quantize(g, F, n, F, wsb + L.gq, L.fkp, wsb + L.gs, L.fkp / 32, s),
                     "gate-product quantization"));
    MxOperand gq;
    gq.data = wsb + L.gq;
    gq.ld = L.fkp;
    gq.scale = wsb + L.gs;
    gq.ld_scale = L.fkp / 32;
    return hip_status(launch_gemm_mx8(EPI_RESIDUAL, gq, wmx(4), MxOperand{}, io->x, io->ld_x,
                                      mslot(5), ldm, n, C, F, s),
                      "swiglu down-projection (fp8)");
  }
  TRY(hip_status(launch_gemm(bf, EPI_SWIGLU, h1, C, w->w1, w->w3, C, g, F, nullptr, 0, n, F, C, s),
                 "swiglu up-projection"));
  // A10 x <- x + gate2 * (g w2^T)
  return hip_status(launch_gemm(bf, EPI_RESIDUAL, g, F, w->w2, nullptr, F, io->x, io->ld_x,
                                mslot(5), ldm, n, C, F, s),
                    "swiglu down-projection");
}

// ------------------------------------------------------------ loop glue

size_t h3_timestep_workspace_size(int32_t dim) {
  return dim > 0 ? (size_t)round_up((int64_t)dim * 4, 256) : 0;
}

h3_status h3_timestep_modulation(float sigma, const void* w_t1, const void* w_t2,
                                 const void* table, void* mod_out, int32_t n_blocks,
                                 int32_t dim, int32_t emb_dim, void* ws, size_t ws_bytes,
                                 h3_dtype dtype, void* stream) {
  g_err[0] = 0;
  TRY(check_dtype(dtype));
  CHECK(std::isfinite(sigma), "sigma must be finite");
  CHECK(dim > 0 && dim % 8 == 0, "dim must be a positive multiple of 8");
  CHECK(emb_dim > 0 && emb_dim % 16 == 0 && emb_dim <= 1024, "emb_dim must be a multiple of 16, <= 1024");
  CHECK(n_blocks > 0, "n_blocks must be positive");
  CHECK(w_t1 && w_t2 && table && mod_out, "NULL tensor");
  CHECK(aligned16(w_t1) && aligned16(w_t2), "weights must be 16-byte aligned");
  if (ws_bytes < h3_timestep_workspace_size(dim))
    return fail(H3_ERR_WORKSPACE, "timestep workspace too small");
  CHECK(ws && aligned16(ws), "workspace is NULL or not 16-byte aligned");
  TRY(check_device());
  return hip_status(launch_timestep(dtype == H3_BF16, sigma, w_t1, w_t2, table, mod_out, n_blocks,
                                    dim, emb_dim, ws, (hipStream_t)stream),
                    "timestep launch");
}

h3_status h3_euler_update(void* z, const void* u, void* x_next, int64_t n, float sigma_from,
                          float sigma_to, h3_dtype dtype, void* stream) {
  g_err[0] = 0;
  TRY(check_dtype(dtype));
  CHECK(n >= 0 && n % 8 == 0, "n must be a non-negative multiple of 8");
  if (n == 0) return H3_OK;
  CHECK(z && u && aligned16(z) && aligned16(u), "z and u must be non-NULL, 16-byte aligned");
  CHECK(!x_next || aligned16(x_next), "x_next must be 16-byte aligned");
  CHECK(std::isfinite(sigma_from) && std::isfinite(sigma_to), "sigmas must be finite");
  TRY(check_device());
  return hip_status(launch_euler(dtype == H3_BF16, z, u, x_next, n, sigma_to - sigma_from,
                                 (hipStream_t)stream),
                    "euler launch");
}

h3_status h3_frames_to_u8(const void* frames, int64_t B, int64_t T, int64_t H, int64_t W,
                          void* out, int32_t layout, void* stream) {
  g_err[0] = 0;
  CHECK(B >= 0 && T >= 0 && H >= 0 && W >= 0, "B, T, H, W must be non-negative");
  CHECK(layout == 0 || layout == 1, "layout must be 0 (BTHWC) or 1 (BTCHW planar)");
  CHECK(W <= ((int64_t)1 << 31) && H <= ((int64_t)1 << 31), "H and W must be below 2^31");
  const double total = 3.0 * (double)B * (double)T * (double)H * (double)W;
  CHECK(total < 9.0e15, "frame tensor too large");
  if (B == 0 || T == 0 || H == 0 || W == 0) return H3_OK;
  CHECK(frames && out && aligned16(frames) && aligned16(out),
        "frames and out must be non-NULL, 16-byte aligned");
  const int64_t n = 3 * B * T * H * W;
  const uintptr_t fa = (uintptr_t)frames, oa = (uintptr_t)out;
  CHECK(oa + (uintptr_t)n <= fa || fa + (uintptr_t)n * 4 <= oa, "frames and out overlap");
  TRY(check_device());
  return hip_status(launch_frames_u8((const float*)frames, (uint8_t*)out, B, T, H, W, layout,
                                     (hipStream_t)stream),
                    "frames launch");
}

}  // extern "C"
