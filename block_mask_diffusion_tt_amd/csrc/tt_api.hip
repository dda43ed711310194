// Host side of the C ABI declared in include/tt.h: argument validation (no
// HIP call happens before every host-visible argument has been checked),
// workspace carving, kernel launches and the block denoising loop.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "../../include/tt.h"
#include "tt_internal.h"

namespace tt {

int device_cus() {
  constexpr int kDefault = 256;   // MI355X
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return kDefault;
  }
  // asked once per device (concurrent first calls store the same value)
  static std::atomic<int> cus[64];
  int n = dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      return kDefault;
    }
    if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace tt

namespace {

thread_local std::string g_err;

tt_status fail(tt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

tt_status ok() {
  g_err.clear();
  return TT_OK;
}

tt_status hip_fail(hipError_t e, const char* what) {
  return fail(TT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elt_size(int dtype) { return dtype == TT_BF16 ? 2 : 4; }

// TT_VALIDATE set (and not "0"): check the context arrays on the device
// before a call's kernels, and wait for the outcome.
bool validate_enabled() {
  const char* v = getenv("TT_VALIDATE");
  return v && v[0] && strcmp(v, "0") != 0;
}

tt_status check_ctx_on_device(const char* fn, int B, const int64_t* ctx_start,
                              const int32_t* ctx_len, const int64_t* ctx_end,
                              const uint8_t* active, tt_stream stream) {
  if (!validate_enabled() || B == 0) return TT_OK;
  int64_t v[4];
  const hipError_t e = tt::validate_ctx(B, ctx_start, ctx_len, ctx_end, active, v,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  if (v[0] < 0) return TT_OK;
  const long long b = v[0], x = v[2], y = v[3];
  switch (v[1]) {
    case 1: return fail(TT_ERR_INVALID_ARG, "%s: TT_VALIDATE: ctx_len[%lld] = %lld < 0", fn, b, x);
    case 2: return fail(TT_ERR_INVALID_ARG, "%s: TT_VALIDATE: ctx_start[%lld] = %lld < 0", fn, b, x);
    case 3:
      return fail(TT_ERR_INVALID_ARG,
                  "%s: TT_VALIDATE: ctx_end[%lld] = %lld is below ctx_start + ctx_len = %lld", fn,
                  b, x, y);
    default:
      return fail(TT_ERR_INVALID_ARG,
                  "%s: TT_VALIDATE: the reserved regions of sequences %lld and %lld overlap", fn, b,
                  x);
  }
}

tt_status check_shape(const tt_attn_shape* s) {
  if (!s) return fail(TT_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 0) return fail(TT_ERR_INVALID_ARG, "batch %d < 0", s->batch);
  if (s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(TT_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", s->n_q_heads,
                s->n_kv_heads);
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(TT_ERR_INVALID_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d",
                s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads > 4096) return fail(TT_ERR_INVALID_ARG, "n_q_heads %d > 4096", s->n_q_heads);
  if (s->head_dim < 1) return fail(TT_ERR_INVALID_ARG, "head_dim %d < 1", s->head_dim);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(TT_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", s->head_dim);
  if (s->block_size < 1 || s->block_size > 64)
    return fail(TT_ERR_INVALID_ARG, "block_size %d outside [1, 64]", s->block_size);
  if (s->dtype != TT_BF16 && s->dtype != TT_F32)
    return fail(TT_ERR_INVALID_ARG, "dtype %d is neither TT_BF16 nor TT_F32", s->dtype);
  return TT_OK;
}

tt_status check_unmask_scalars(int32_t batch, int32_t S, int32_t V, int64_t row_stride,
                               float gamma, float temperature) {
  if (batch < 0) return fail(TT_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (S < 1 || S > 64) return fail(TT_ERR_INVALID_ARG, "block_size %d outside [1, 64]", S);
  if (V < 1) return fail(TT_ERR_INVALID_ARG, "vocab %d < 1", V);
  if (row_stride < V)
    return fail(TT_ERR_INVALID_ARG, "row_stride %lld < vocab %d", (long long)row_stride, V);
  if (isnan(gamma)) return fail(TT_ERR_INVALID_ARG, "gamma is NaN");
  if (!(temperature >= 1e-30f) || isinf(temperature))
    return fail(TT_ERR_INVALID_ARG, "temperature %g must be finite and >= 1e-30", temperature);
  return TT_OK;
}

// Hands out 256-byte-aligned pieces of a workspace in order.  With a NULL
// base it only counts (a size query), without forming pointers from NULL.
struct Carver {
  char* base;
  size_t off = 0;
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += tt::align_up(bytes, 256);
    return p;
  }
};

size_t denoise_bytes(const tt_attn_shape* s, int n_layers, int max_ctx_len, int vocab) {
  const size_t B = s->batch, S = s->block_size, Hq = s->n_q_heads, Hkv = s->n_kv_heads,
               d = s->head_dim, e = elt_size(s->dtype), W = Hq * d;
  size_t t = 0;
  auto add = [&](size_t b) { t += tt::align_up(b, 256); };
  add(static_cast<size_t>(n_layers) * 3 * B * W * 4);  // ada
  add(B * TT_TIMESTEP_DIM * 4);                          // emb
  add(B * S * Hq * d * e);                               // q
  add(B * S * Hkv * d * e);                              // k
  add(B * S * Hkv * d * e);                              // v
  add(B * S * Hq * d * e);                               // out
  add(B * S * static_cast<size_t>(vocab) * e);           // logits
  add(B * 4);                                            // n_masked
  add(B);                                                // active
  add(4);                                                // total
  const tt::AttnPlan ap = tt::attn_plan(s->batch, s->block_size, s->n_q_heads, s->n_kv_heads,
                                        s->head_dim, s->dtype, max_ctx_len);
  add(ap.total_bytes);
  const tt::UnmaskPlan up = tt::unmask_plan(s->batch, s->block_size, vocab);
  add(up.total_bytes);
  return t;
}

}  // namespace

extern "C" {

const char* tt_last_error(void) { return g_err.c_str(); }

int tt_abi_version(void) { return TT_ABI_VERSION; }

size_t tt_block_attn_workspace_size(const tt_attn_shape* shape, int32_t max_ctx_len) {
  if (check_shape(shape) != TT_OK) return 0;
  if (max_ctx_len < 0) {
    fail(TT_ERR_INVALID_ARG, "max_ctx_len %d < 0", max_ctx_len);
    return 0;
  }
  ok();
  const tt::AttnPlan p = tt::attn_plan(shape->batch, shape->block_size, shape->n_q_heads,
                                       shape->n_kv_heads, shape->head_dim, shape->dtype,
                                       max_ctx_len);
  return p.total_bytes < 256 ? 256 : p.total_bytes;
}

}  // extern "C"

// ------------------------------------------------- allocation-free attention
// Workspace of tt_block_attn_noalloc: one array in every GPU's memory, held
// by the library until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in); it uses the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[TT_BLOCK_ATTN_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up once per
// device, with that device current); NULL after a failure, reported in *e.
void* scratch_of_current_device(hipError_t* e) {
  int dev = 0;
  *e = hipGetDevice(&dev);
  if (*e != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *e = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    *e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*e != hipSuccess || !p) {
      if (*e == hipSuccess) *e = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Validation and launch shared by the denoiser's and the context tower's
// attention calls.  use_scratch: the workspace is this device's `scratch`
// (looked up after every argument has been checked).
tt_status block_attn_common(const char* fn, const tt_attn_shape* shape, const void* q_blk,
                            const void* k_blk, const void* v_blk, const void* k_ctx,
                            const void* v_ctx, const int64_t* ctx_start, const int32_t* ctx_len,
                            const int64_t* ctx_end, int32_t max_ctx_len, const uint8_t* active,
                            const float* ada_shift, const float* ada_scale, const float* ada_gate,
                            const void* residual, void* out, float* lse, int causal,
                            void* workspace, size_t workspace_bytes, tt_stream stream,
                            bool use_scratch = false) {
  tt_status st = check_shape(shape);
  if (st != TT_OK) return st;
  if (max_ctx_len < 0) return fail(TT_ERR_INVALID_ARG, "%s: max_ctx_len %d < 0", fn, max_ctx_len);
  if (!q_blk || !k_blk || !v_blk || !out)
    return fail(TT_ERR_INVALID_ARG, "%s: q_blk, k_blk, v_blk and out must be non-NULL", fn);
  if (!k_ctx || !v_ctx || !ctx_start || !ctx_len)
    return fail(TT_ERR_INVALID_ARG, "%s: k_ctx, v_ctx, ctx_start and ctx_len must be non-NULL", fn);
  const void* tensors[] = {q_blk, k_blk, v_blk, k_ctx, v_ctx, out, residual};
  for (const void* t : tensors)
    if (t && !aligned(t, 16))
      return fail(TT_ERR_INVALID_ARG,
                  "%s: q/k/v/context/out/residual buffers must be 16-byte aligned", fn);
  const void* ada[] = {ada_shift, ada_scale, ada_gate};
  for (const void* t : ada)
    if (t && !aligned(t, 16))
      return fail(TT_ERR_INVALID_ARG, "%s: ada_shift/ada_scale/ada_gate must be 16-byte aligned", fn);
  if (!aligned(ctx_start, 8) || !aligned(ctx_len, 4) || (lse && !aligned(lse, 4)) ||
      (ctx_end && !aligned(ctx_end, 8)))
    return fail(TT_ERR_INVALID_ARG, "%s: misaligned ctx_start/ctx_end/ctx_len/lse buffer", fn);
  if (shape->batch == 0) return ok();
  const tt::AttnPlan p = tt::attn_plan(shape->batch, shape->block_size, shape->n_q_heads,
                                       shape->n_kv_heads, shape->head_dim, shape->dtype,
                                       max_ctx_len);
  if (use_scratch) {
    if (p.total_bytes > TT_BLOCK_ATTN_SCRATCH_BYTES)
      return fail(TT_ERR_WORKSPACE, "%s: the launch needs %zu bytes of workspace, more than the "
                  "%llu-byte scratch; use tt_block_attn with a workspace", fn, p.total_bytes,
                  static_cast<unsigned long long>(TT_BLOCK_ATTN_SCRATCH_BYTES));
    hipError_t se = hipSuccess;
    workspace = scratch_of_current_device(&se);
    if (!workspace) return hip_fail(se, fn);
    workspace_bytes = TT_BLOCK_ATTN_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < p.total_bytes)
    return fail(TT_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes,
                p.total_bytes);
  if (!aligned(workspace, 256))
    return fail(TT_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  tt::AttnArgs a{};
  a.B = shape->batch; a.S = shape->block_size; a.Hq = shape->n_q_heads;
  a.Hkv = shape->n_kv_heads; a.d = shape->head_dim; a.dtype = shape->dtype;
  a.q = q_blk; a.kb = k_blk; a.vb = v_blk; a.kc = k_ctx; a.vc = v_ctx;
  a.ctx_start = ctx_start; a.ctx_len = ctx_len; a.active = active;
  a.shift = ada_shift; a.scale = ada_scale; a.gate = ada_gate;
  a.residual = residual; a.out = out; a.lse = lse;
  a.causal = causal;
  a.ctx_end = ctx_end;
  a.kc_out = const_cast<void*>(k_ctx);
  a.vc_out = const_cast<void*>(v_ctx);
  st = check_ctx_on_device(fn, shape->batch, ctx_start, ctx_len, ctx_end, active, stream);
  if (st != TT_OK) return st;
  const hipError_t e = tt::launch_block_attn(a, p, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // namespace

extern "C" {

tt_status tt_block_attn(const tt_attn_shape* shape, const void* q_blk, const void* k_blk,
                        const void* v_blk, const void* k_ctx, const void* v_ctx,
                        const int64_t* ctx_start, const int32_t* ctx_len, int32_t max_ctx_len,
                        const uint8_t* active, const float* ada_shift, const float* ada_scale,
                        const float* ada_gate, const void* residual, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, tt_stream stream) {
  return block_attn_common("tt_block_attn", shape, q_blk, k_blk, v_blk, k_ctx, v_ctx, ctx_start,
                           ctx_len, nullptr, max_ctx_len, active, ada_shift, ada_scale, ada_gate,
                           residual, out, lse, 0, workspace, workspace_bytes, stream);
}

tt_status tt_ctx_block_attn(const tt_attn_shape* shape, const void* q_blk, const void* k_blk,
                            const void* v_blk, void* k_ctx, void* v_ctx,
                            const int64_t* ctx_start, const int32_t* ctx_len,
                            const int64_t* ctx_end, int32_t max_ctx_len, const uint8_t* active,
                            const void* residual, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, tt_stream stream) {
  return block_attn_common("tt_ctx_block_attn", shape, q_blk, k_blk, v_blk, k_ctx, v_ctx,
                           ctx_start, ctx_len, ctx_end, max_ctx_len, active, nullptr, nullptr,
                           nullptr, residual, out, lse, 1, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" {

tt_status tt_block_attn_noalloc(const tt_attn_shape* shape, const void* q_blk, const void* k_blk,
                                const void* v_blk, const void* k_ctx, const void* v_ctx,
                                const int64_t* ctx_start, const int32_t* ctx_len,
                                int32_t max_ctx_len, const uint8_t* active,
                                const float* ada_shift, const float* ada_scale,
                                const float* ada_gate, const void* residual, void* out,
                                float* lse, tt_stream stream) {
  return block_attn_common("tt_block_attn_noalloc", shape, q_blk, k_blk, v_blk, k_ctx, v_ctx,
                           ctx_start, ctx_len, nullptr, max_ctx_len, active, ada_shift, ada_scale,
                           ada_gate, residual, out, lse, 0, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {

tt_status check_mamba_shape(const char* fn, const tt_mamba_shape* shape) {
  if (!shape) return fail(TT_ERR_INVALID_ARG, "%s: shape is NULL", fn);
  const tt_mamba_shape& m = *shape;
  if (m.batch < 0 || m.n_heads < 1 || m.n_groups < 1 || m.head_dim < 1 || m.d_state < 1)
    return fail(TT_ERR_INVALID_ARG, "%s: bad sizes (B=%d H=%d G=%d P=%d N=%d)", fn, m.batch,
                m.n_heads, m.n_groups, m.head_dim, m.d_state);
  if (m.n_heads % m.n_groups != 0)
    return fail(TT_ERR_INVALID_ARG, "%s: n_groups %d does not divide n_heads %d", fn, m.n_groups,
                m.n_heads);
  if (m.conv_width < 2 || m.conv_width > 8)
    return fail(TT_ERR_INVALID_ARG, "%s: conv_width %d outside [2, 8]", fn, m.conv_width);
  if (m.block_size < 1 || m.block_size > 64)
    return fail(TT_ERR_INVALID_ARG, "%s: block_size %d outside [1, 64]", fn, m.block_size);
  if (m.dtype != TT_BF16 && m.dtype != TT_F32)
    return fail(TT_ERR_INVALID_ARG, "%s: dtype %d is neither TT_BF16 nor TT_F32", fn, m.dtype);
  if (m.conv_width > 4)
    return fail(TT_ERR_UNSUPPORTED, "%s: conv_width %d not supported (2 to 4)", fn, m.conv_width);
  if (!tt::mamba_supported(m.head_dim, m.d_state, m.conv_width))
    return fail(TT_ERR_UNSUPPORTED, "%s: head_dim %d / d_state %d not supported (32 or 64 / 64 or 128)",
                fn, m.head_dim, m.d_state);
  if (static_cast<int64_t>(m.n_heads) * m.head_dim + 2LL * m.n_groups * m.d_state > INT32_MAX / 64)
    return fail(TT_ERR_INVALID_ARG, "%s: too many channels", fn);
  if (tt::mamba_lds_bytes(m.block_size, m.head_dim, m.d_state) > 160 * 1024 ||
      tt::mamba_group_lds_bytes(m.block_size, m.d_state) > 160 * 1024)
    return fail(TT_ERR_UNSUPPORTED, "%s: block too long for the LDS staging", fn);
  return TT_OK;
}

}  // namespace

extern "C" {

size_t tt_mamba_workspace_size(const tt_mamba_shape* shape) {
  if (check_mamba_shape("tt_mamba_workspace_size", shape) != TT_OK) return 0;
  ok();
  const size_t n = tt::mamba_workspace_bytes(shape->batch, shape->block_size, shape->n_groups,
                                             shape->d_state);
  return n < 256 ? 256 : n;
}

tt_status tt_mamba_block_scan(const tt_mamba_shape* shape, const void* xbc, const float* dt_raw,
                              const void* conv_state, const float* ssm_state,
                              const float* conv_w, const float* conv_b, const float* A_log,
                              const float* dt_bias, const float* D, const uint8_t* active,
                              void* y, void* conv_state_out, float* ssm_state_out,
                              void* workspace, size_t workspace_bytes, tt_stream stream) {
  const char* fn = "tt_mamba_block_scan";
  tt_status cs = check_mamba_shape(fn, shape);
  if (cs != TT_OK) return cs;
  const tt_mamba_shape& m = *shape;
  if (!xbc || !dt_raw || !conv_state || !ssm_state || !conv_w || !A_log || !y)
    return fail(TT_ERR_INVALID_ARG, "%s: xbc, dt_raw, conv_state, ssm_state, conv_w, A_log and y must be non-NULL", fn);
  if (!aligned(ssm_state, 16) || (ssm_state_out && !aligned(ssm_state_out, 16)))
    return fail(TT_ERR_INVALID_ARG, "%s: ssm_state buffers must be 16-byte aligned", fn);
  const size_t e = elt_size(m.dtype);
  const void* ptrs[] = {xbc, conv_state, y, conv_state_out};
  for (const void* t : ptrs)
    if (t && !aligned(t, e)) return fail(TT_ERR_INVALID_ARG, "%s: misaligned xbc/conv_state/y buffer", fn);
  if (!aligned(y, 4 * e))
    return fail(TT_ERR_INVALID_ARG, "%s: y must be aligned to 4 elements (%zu bytes)", fn, 4 * e);
  const void* fptrs[] = {dt_raw, conv_w, conv_b, A_log, dt_bias, D};
  for (const void* t : fptrs)
    if (t && !aligned(t, 4)) return fail(TT_ERR_INVALID_ARG, "%s: misaligned fp32 parameter", fn);
  if (conv_state_out) {
    const size_t C = static_cast<size_t>(m.n_heads) * m.head_dim + 2 * static_cast<size_t>(m.n_groups) * m.d_state;
    const size_t bytes = static_cast<size_t>(m.batch) * C * (m.conv_width - 1) * e;
    const char* a0 = static_cast<const char*>(conv_state);
    const char* b0 = static_cast<const char*>(conv_state_out);
    if (a0 < b0 + bytes && b0 < a0 + bytes)
      return fail(TT_ERR_INVALID_ARG, "%s: conv_state_out overlaps conv_state", fn);
  }
  if (m.batch == 0) return ok();
  const size_t need = tt::mamba_workspace_bytes(m.batch, m.block_size, m.n_groups, m.d_state);
  if (!workspace || workspace_bytes < need)
    return fail(TT_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(TT_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  tt::MambaArgs a{};
  a.B = m.batch; a.S = m.block_size; a.H = m.n_heads; a.P = m.head_dim; a.N = m.d_state;
  a.G = m.n_groups; a.W = m.conv_width; a.dtype = m.dtype;
  a.xbc = xbc; a.dt_raw = dt_raw; a.conv_state = conv_state; a.ssm_state = ssm_state;
  a.conv_w = conv_w; a.conv_b = conv_b; a.A_log = A_log; a.dt_bias = dt_bias; a.D = D;
  a.active = active; a.y = y; a.conv_state_out = conv_state_out; a.ssm_state_out = ssm_state_out;
  const hipError_t he = tt::launch_mamba_scan(a, workspace, static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, fn);
  return ok();
}

tt_status tt_ctx_advance(int32_t batch, int32_t block_size, const int64_t* ctx_start,
                         const int64_t* ctx_end, int32_t* ctx_len, const uint8_t* active,
                         uint8_t* appended, tt_stream stream) {
  if (batch < 0) return fail(TT_ERR_INVALID_ARG, "tt_ctx_advance: batch %d < 0", batch);
  if (block_size < 1 || block_size > 64)
    return fail(TT_ERR_INVALID_ARG, "tt_ctx_advance: block_size %d outside [1, 64]", block_size);
  if (!ctx_start || !ctx_end || !ctx_len)
    return fail(TT_ERR_INVALID_ARG, "tt_ctx_advance: ctx_start, ctx_end and ctx_len must be non-NULL");
  if (!aligned(ctx_start, 8) || !aligned(ctx_end, 8) || !aligned(ctx_len, 4))
    return fail(TT_ERR_INVALID_ARG, "tt_ctx_advance: misaligned ctx_start/ctx_end/ctx_len");
  if (batch == 0) return ok();
  const tt_status vs = check_ctx_on_device("tt_ctx_advance", batch, ctx_start, ctx_len, ctx_end,
                                           active, stream);
  if (vs != TT_OK) return vs;
  const hipError_t e = tt::launch_ctx_advance(batch, block_size, ctx_start, ctx_end, ctx_len,
                                              active, appended, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tt_ctx_advance launch");
  return ok();
}

tt_status tt_workspace_clear(void* workspace, size_t bytes, tt_stream stream) {
  if (bytes == 0) return ok();
  if (!workspace) return fail(TT_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(TT_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const hipError_t e = tt::launch_clear(workspace, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tt_workspace_clear launch");
  return ok();
}

tt_status tt_timestep_embed(int32_t batch, const float* t, float* emb, tt_stream stream) {
  if (batch < 0) return fail(TT_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (!t || !emb) return fail(TT_ERR_INVALID_ARG, "t and emb must be non-NULL");
  if (batch == 0) return ok();
  const hipError_t e =
      tt::launch_timestep_embed(batch, t, nullptr, 1, emb, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tt_timestep_embed launch");
  return ok();
}

tt_status tt_adaln_single(int32_t batch, int32_t width, int32_t n_layers, const float* t_emb,
                          const void* w, const float* bias, const float* table, float* ada,
                          tt_stream stream) {
  if (batch < 0) return fail(TT_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (width < 4 || width % 4 != 0)
    return fail(TT_ERR_INVALID_ARG, "width %d must be a positive multiple of 4", width);
  if (n_layers < 1) return fail(TT_ERR_INVALID_ARG, "n_layers %d < 1", n_layers);
  if (!t_emb || !w || !ada) return fail(TT_ERR_INVALID_ARG, "t_emb, w and ada must be non-NULL");
  if (!aligned(w, 8) || !aligned(t_emb, 4) || !aligned(ada, 16) || !aligned(bias, 16) ||
      !aligned(table, 16))
    return fail(TT_ERR_INVALID_ARG,
                "misaligned adaLN buffer (w needs 8 bytes; ada, bias and table 16)");
  if (batch == 0) return ok();
  const hipError_t e = tt::launch_adaln_single(batch, width, n_layers, t_emb, w, bias, table, ada,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tt_adaln_single launch");
  return ok();
}

size_t tt_unmask_workspace_size(int32_t batch, int32_t block_size, int32_t vocab) {
  if (check_unmask_scalars(batch, block_size, vocab, vocab, 0.f, 1.f) != TT_OK) return 0;
  ok();
  const tt::UnmaskPlan p = tt::unmask_plan(batch, block_size, vocab);
  return p.total_bytes < 256 ? 256 : p.total_bytes;
}

}  // extern "C"

namespace {

tt_status unmask_common(const char* fn, int32_t batch, int32_t block_size, int32_t vocab,
                        const void* logits, int32_t dtype, int64_t row_stride, float gamma,
                        float temperature, int sample, uint64_t seed, int32_t block_index,
                        int32_t mask_token_id, int32_t step, int32_t* tokens, uint8_t* masked,
                        uint8_t* committed_now, float* conf, int32_t* pred, int8_t* commit_step,
                        int32_t* n_masked, void* workspace, size_t workspace_bytes,
                        tt_stream stream) {
  tt_status st = check_unmask_scalars(batch, block_size, vocab, row_stride, gamma, temperature);
  if (st != TT_OK) return st;
  if (dtype != TT_BF16 && dtype != TT_F32)
    return fail(TT_ERR_INVALID_ARG, "%s: dtype %d is neither TT_BF16 nor TT_F32", fn, dtype);
  if (!logits || !tokens || !masked)
    return fail(TT_ERR_INVALID_ARG, "%s: logits, tokens and masked must be non-NULL", fn);
  if (sample && (step < 0 || block_index < 0))
    return fail(TT_ERR_INVALID_ARG, "%s: step %d and block_index %d must be >= 0", fn, step,
                block_index);
  if (!aligned(logits, elt_size(dtype)) || !aligned(tokens, 4) || (conf && !aligned(conf, 4)) ||
      (pred && !aligned(pred, 4)) || (n_masked && !aligned(n_masked, 4)))
    return fail(TT_ERR_INVALID_ARG, "%s: misaligned unmasking buffer", fn);
  if (batch == 0) return ok();
  const tt::UnmaskPlan p = tt::unmask_plan(batch, block_size, vocab);
  if (!workspace || workspace_bytes < p.total_bytes)
    return fail(TT_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes,
                p.total_bytes);
  if (!aligned(workspace, 16))
    return fail(TT_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  tt::UnmaskArgs a{};
  a.B = batch; a.S = block_size; a.V = vocab; a.dtype = dtype;
  a.logits = logits; a.row_stride = row_stride; a.gamma = gamma; a.temperature = temperature;
  a.mask_id = mask_token_id; a.step = step; a.tokens = tokens; a.masked = masked;
  a.committed_now = committed_now; a.conf = conf; a.pred = pred; a.commit_step = commit_step;
  a.n_masked = n_masked;
  a.sample = sample; a.seed = seed; a.block_index = block_index;
  const hipError_t e =
      tt::launch_confidence_unmask(a, p, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // namespace

extern "C" {

tt_status tt_confidence_unmask(int32_t batch, int32_t block_size, int32_t vocab,
                               const void* logits, int32_t dtype, int64_t row_stride, float gamma,
                               float temperature, int32_t mask_token_id, int32_t step,
                               int32_t* tokens, uint8_t* masked, uint8_t* committed_now,
                               float* conf, int32_t* pred, int8_t* commit_step,
                               int32_t* n_masked, void* workspace, size_t workspace_bytes,
                               tt_stream stream) {
  return unmask_common("tt_confidence_unmask", batch, block_size, vocab, logits, dtype, row_stride,
                       gamma, temperature, 0, 0, 0, mask_token_id, step, tokens, masked,
                       committed_now, conf, pred, commit_step, n_masked, workspace,
                       workspace_bytes, stream);
}

tt_status tt_sample_unmask(int32_t batch, int32_t block_size, int32_t vocab, const void* logits,
                           int32_t dtype, int64_t row_stride, float gamma, float temperature,
                           uint64_t seed, int32_t block_index, int32_t mask_token_id,
                           int32_t step, int32_t* tokens, uint8_t* masked,
                           uint8_t* committed_now, float* conf, int32_t* pred,
                           int8_t* commit_step, int32_t* n_masked, void* workspace,
                           size_t workspace_bytes, tt_stream stream) {
  return unmask_common("tt_sample_unmask", batch, block_size, vocab, logits, dtype, row_stride,
                       gamma, temperature, 1, seed, block_index, mask_token_id, step, tokens,
                       masked, committed_now, conf, pred, commit_step, n_masked, workspace,
                       workspace_bytes, stream);
}

size_t tt_denoise_workspace_size(const tt_attn_shape* shape, int32_t n_layers,
                                 int32_t max_ctx_len, int32_t vocab) {
  if (check_shape(shape) != TT_OK) return 0;
  if (n_layers < 1 || max_ctx_len < 0 || vocab < 1) {
    fail(TT_ERR_INVALID_ARG, "n_layers %d, max_ctx_len %d, vocab %d", n_layers, max_ctx_len, vocab);
    return 0;
  }
  ok();
  return denoise_bytes(shape, n_layers, max_ctx_len, vocab);
}

}  // extern "C"

namespace {

// The workspace buffers of the denoising loop, carved in denoise_bytes order.
struct DenoiseBufs {
  float* ada; float* emb;
  void* q; void* kb; void* vb; void* out; void* logits;
  int32_t* n_masked; uint8_t* active; int32_t* total;
  void* attn_ws; void* unmask_ws;
  tt::AttnPlan ap; tt::UnmaskPlan up;
};

DenoiseBufs carve_denoise(Carver& cv, const tt_attn_shape* shape, int n_layers, int max_ctx_len,
                          int vocab) {
  const size_t B = shape->batch, S = shape->block_size, Hq = shape->n_q_heads,
               Hkv = shape->n_kv_heads, d = shape->head_dim, e = elt_size(shape->dtype),
               W = Hq * d;
  DenoiseBufs z{};
  z.ada = static_cast<float*>(cv.take(static_cast<size_t>(n_layers) * 3 * B * W * 4));
  z.emb = static_cast<float*>(cv.take(B * TT_TIMESTEP_DIM * 4));
  z.q = cv.take(B * S * Hq * d * e);
  z.kb = cv.take(B * S * Hkv * d * e);
  z.vb = cv.take(B * S * Hkv * d * e);
  z.out = cv.take(B * S * Hq * d * e);
  z.logits = cv.take(B * S * static_cast<size_t>(vocab) * e);
  z.n_masked = static_cast<int32_t*>(cv.take(B * 4));
  z.active = static_cast<uint8_t*>(cv.take(B));
  z.total = static_cast<int32_t*>(cv.take(4));
  z.ap = tt::attn_plan(shape->batch, shape->block_size, shape->n_q_heads, shape->n_kv_heads,
                       shape->head_dim, shape->dtype, max_ctx_len);
  z.attn_ws = cv.take(z.ap.total_bytes);
  z.up = tt::unmask_plan(shape->batch, shape->block_size, vocab);
  z.unmask_ws = cv.take(z.up.total_bytes);
  return z;
}

struct LoopOpts {
  int first_step;     // absolute index of the loop's first step
  int n_layers, max_steps, vocab, mask_id;
  float gamma, temperature;
  int sample; uint64_t seed; int block;
  int finish_block;   // the last allowed step commits every masked slot
};

// The block denoising loop (tt_denoise_block, and each block of tt_generate):
// per step, the active set and the masked count (one wait on the stream),
// adaLN vectors, the layers' attention and the unmasking pass.  The
// callables fill the provider's buffers: layer_inputs(step, layer, prev_out)
// and logits(step) return the callback's status.
template <typename LayerFn, typename LogitsFn>
tt_status denoise_loop(const char* fn, const tt_attn_shape* shape, const LoopOpts& o,
                       const void* const* k_ctx_layers, const void* const* v_ctx_layers,
                       const int64_t* ctx_start, const int32_t* ctx_len, const void* ada_w,
                       const float* ada_bias, const float* ada_table, LayerFn&& layer_inputs,
                       LogitsFn&& logits_fn, int32_t* tokens, uint8_t* masked,
                       int8_t* commit_step, int32_t* steps_taken, const DenoiseBufs& z,
                       tt_stream stream) {
  const int B = shape->batch, S = shape->block_size, Hq = shape->n_q_heads,
            Hkv = shape->n_kv_heads, d = shape->head_dim;
  const size_t W = static_cast<size_t>(Hq) * d;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t he = tt::launch_count_masked(B, S, masked, z.n_masked, hs);
  if (he != hipSuccess) return hip_fail(he, fn);
  const int k_end = o.first_step + o.max_steps;
  for (int k = o.first_step; k < k_end; ++k) {
    he = tt::launch_active_from_masked(B, z.n_masked, z.active, z.total, hs);
    if (he != hipSuccess) return hip_fail(he, fn);
    int32_t host_total = 0;
    he = hipMemcpyAsync(&host_total, z.total, sizeof(int32_t), hipMemcpyDeviceToHost, hs);
    if (he == hipSuccess) he = hipStreamSynchronize(hs);
    if (he != hipSuccess) return hip_fail(he, fn);
    if (host_total == 0) break;
    if (ada_w) {
      he = tt::launch_timestep_embed(B, nullptr, z.n_masked, S, z.emb, hs);
      if (he == hipSuccess)
        he = tt::launch_adaln_single(B, static_cast<int>(W), o.n_layers, z.emb, ada_w, ada_bias,
                                     ada_table, z.ada, hs);
      if (he != hipSuccess) return hip_fail(he, fn);
    }
    for (int l = 0; l < o.n_layers; ++l) {
      const int rc = layer_inputs(k, l, l == 0 ? nullptr : z.out);
      if (rc != 0)
        return fail(TT_ERR_CALLBACK, "%s: layer_inputs(step %d, layer %d) returned %d", fn, k, l, rc);
      tt::AttnArgs a{};
      a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.dtype = shape->dtype;
      a.q = z.q; a.kb = z.kb; a.vb = z.vb; a.kc = k_ctx_layers[l]; a.vc = v_ctx_layers[l];
      a.ctx_start = ctx_start; a.ctx_len = ctx_len; a.active = z.active;
      if (ada_w) {
        a.shift = z.ada + (static_cast<size_t>(l) * 3 + 0) * B * W;
        a.scale = z.ada + (static_cast<size_t>(l) * 3 + 1) * B * W;
        a.gate = z.ada + (static_cast<size_t>(l) * 3 + 2) * B * W;
      }
      a.residual = nullptr; a.out = z.out; a.lse = nullptr;
      he = tt::launch_block_attn(a, z.ap, z.attn_ws, hs);
      if (he != hipSuccess) return hip_fail(he, fn);
    }
    const int rc = logits_fn(k);
    if (rc != 0) return fail(TT_ERR_CALLBACK, "%s: logits(step %d) returned %d", fn, k, rc);
    tt::UnmaskArgs ua{};
    ua.B = B; ua.S = S; ua.V = o.vocab; ua.dtype = shape->dtype; ua.logits = z.logits;
    ua.row_stride = o.vocab;
    ua.gamma = (o.finish_block && k == k_end - 1) ? -INFINITY : o.gamma;
    ua.temperature = o.temperature;
    ua.mask_id = o.mask_id; ua.step = k; ua.tokens = tokens; ua.masked = masked;
    ua.commit_step = commit_step; ua.n_masked = z.n_masked;
    ua.sample = o.sample; ua.seed = o.seed; ua.block_index = o.block;
    he = tt::launch_confidence_unmask(ua, z.up, z.unmask_ws, hs);
    if (he != hipSuccess) return hip_fail(he, fn);
    if (steps_taken) *steps_taken = k + 1 - o.first_step;
  }
  return TT_OK;
}

tt_status check_layers(const char* fn, int n_layers, const void* const* k_layers,
                       const void* const* v_layers) {
  if (!k_layers || !v_layers)
    return fail(TT_ERR_INVALID_ARG, "%s: k_ctx_layers and v_ctx_layers must be non-NULL", fn);
  for (int l = 0; l < n_layers; ++l) {
    if (!k_layers[l] || !v_layers[l])
      return fail(TT_ERR_INVALID_ARG, "%s: context cache of layer %d is NULL", fn, l);
    if (!aligned(k_layers[l], 16) || !aligned(v_layers[l], 16))
      return fail(TT_ERR_INVALID_ARG, "%s: context cache of layer %d is not 16-byte aligned", fn, l);
  }
  return TT_OK;
}

tt_status check_ada(const char* fn, const tt_attn_shape* shape, const void* ada_w,
                    const float* ada_bias, const float* ada_table) {
  if (ada_w && (shape->n_q_heads * shape->head_dim) % 4 != 0)
    return fail(TT_ERR_INVALID_ARG, "%s: adaLN width must be a multiple of 4", fn);
  if (ada_w && !aligned(ada_w, 8)) return fail(TT_ERR_INVALID_ARG, "%s: ada_w must be 8-byte aligned", fn);
  if (ada_w && (!aligned(ada_bias, 16) || !aligned(ada_table, 16)))
    return fail(TT_ERR_INVALID_ARG, "%s: ada_bias and ada_table must be 16-byte aligned", fn);
  return TT_OK;
}

size_t generate_bytes(const tt_attn_shape* s, int n_layers, int n_blocks, int max_ctx_len,
                      int vocab) {
  const size_t B = s->batch, S = s->block_size;
  size_t t = denoise_bytes(s, n_layers, max_ctx_len + n_blocks * s->block_size, vocab);
  t += tt::align_up(B * S * 4, 256);   // tokens of the block
  t += tt::align_up(B * S, 256);       // masked
  t += tt::align_up(B, 256);           // unfinished
  t += tt::align_up(B, 256);           // appended
  return t;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

tt_status denoise_common(const char* fn, const tt_attn_shape* shape, int32_t n_layers,
                         int32_t first_step, int32_t max_steps, float gamma, float temperature,
                         int32_t sample, uint64_t seed, int32_t block_index,
                         int32_t mask_token_id, int32_t vocab, const void* const* k_ctx_layers,
                         const void* const* v_ctx_layers, const int64_t* ctx_start,
                         const int32_t* ctx_len, int32_t max_ctx_len, const void* ada_w,
                         const float* ada_bias, const float* ada_table,
                         const tt_step_provider* provider, int32_t* tokens, uint8_t* masked,
                         int8_t* commit_step, int32_t* steps_taken, void* workspace,
                         size_t workspace_bytes, tt_stream stream) {
  if (steps_taken) *steps_taken = 0;
  tt_status st = check_shape(shape);
  if (st != TT_OK) return st;
  const int S = shape->block_size;
  if (n_layers < 1) return fail(TT_ERR_INVALID_ARG, "%s: n_layers %d < 1", fn, n_layers);
  if (first_step < 0 || first_step > S)
    return fail(TT_ERR_INVALID_ARG, "%s: first_step %d outside [0, block_size=%d]", fn, first_step, S);
  if (max_steps < 0 || max_steps > S - first_step)
    return fail(TT_ERR_INVALID_ARG, "%s: max_steps %d outside [0, block_size - first_step = %d]", fn,
                max_steps, S - first_step);
  if (sample && block_index < 0)
    return fail(TT_ERR_INVALID_ARG, "%s: block_index %d < 0", fn, block_index);
  if (max_ctx_len < 0) return fail(TT_ERR_INVALID_ARG, "%s: max_ctx_len %d < 0", fn, max_ctx_len);
  st = check_unmask_scalars(shape->batch, S, vocab, vocab, gamma, temperature);
  if (st != TT_OK) return st;
  st = check_layers(fn, n_layers, k_ctx_layers, v_ctx_layers);
  if (st != TT_OK) return st;
  if (!ctx_start || !ctx_len) return fail(TT_ERR_INVALID_ARG, "%s: ctx_start and ctx_len must be non-NULL", fn);
  if (!provider || !provider->layer_inputs || !provider->logits)
    return fail(TT_ERR_INVALID_ARG, "%s: provider and both of its callbacks must be non-NULL", fn);
  if (!tokens || !masked) return fail(TT_ERR_INVALID_ARG, "%s: tokens and masked must be non-NULL", fn);
  st = check_ada(fn, shape, ada_w, ada_bias, ada_table);
  if (st != TT_OK) return st;
  if (shape->batch == 0 || max_steps == 0) return ok();
  const size_t need = denoise_bytes(shape, n_layers, max_ctx_len, vocab);
  if (!workspace || workspace_bytes < need)
    return fail(TT_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(TT_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);

  st = check_ctx_on_device(fn, shape->batch, ctx_start, ctx_len, nullptr, nullptr, stream);
  if (st != TT_OK) return st;
  Carver cv{static_cast<char*>(workspace)};
  const DenoiseBufs z = carve_denoise(cv, shape, n_layers, max_ctx_len, vocab);
  LoopOpts o{};
  o.first_step = first_step;
  o.n_layers = n_layers; o.max_steps = max_steps; o.vocab = vocab; o.mask_id = mask_token_id;
  o.gamma = gamma; o.temperature = temperature;
  o.sample = sample != 0; o.seed = seed; o.block = block_index;
  auto layer_inputs = [&](int k, int l, const void* prev) {
    return provider->layer_inputs(provider->user, k, l, prev, z.q, z.kb, z.vb, stream);
  };
  auto logits_fn = [&](int k) { return provider->logits(provider->user, k, z.out, z.logits, stream); };
  st = denoise_loop(fn, shape, o, k_ctx_layers, v_ctx_layers, ctx_start, ctx_len, ada_w, ada_bias,
                    ada_table, layer_inputs, logits_fn, tokens, masked, commit_step, steps_taken, z,
                    stream);
  if (st != TT_OK) return st;
  const hipError_t he = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, fn);
  return ok();
}

}  // namespace

extern "C" {

tt_status tt_denoise_block(const tt_attn_shape* shape, int32_t n_layers, int32_t max_steps,
                           float gamma, float temperature, int32_t mask_token_id, int32_t vocab,
                           const void* const* k_ctx_layers, const void* const* v_ctx_layers,
                           const int64_t* ctx_start, const int32_t* ctx_len, int32_t max_ctx_len,
                           const void* ada_w, const float* ada_bias, const float* ada_table,
                           const tt_step_provider* provider, int32_t* tokens, uint8_t* masked,
                           int8_t* commit_step, int32_t* steps_taken, void* workspace,
                           size_t workspace_bytes, tt_stream stream) {
  return denoise_common("tt_denoise_block", shape, n_layers, 0, max_steps, gamma, temperature, 0,
                        0, 0, mask_token_id, vocab, k_ctx_layers, v_ctx_layers, ctx_start,
                        ctx_len, max_ctx_len, ada_w, ada_bias, ada_table, provider, tokens, masked,
                        commit_step, steps_taken, workspace, workspace_bytes, stream);
}

tt_status tt_denoise_block_resume(const tt_attn_shape* shape, int32_t n_layers,
                                  int32_t first_step, int32_t max_steps, float gamma,
                                  float temperature, int32_t sample, uint64_t seed,
                                  int32_t block_index, int32_t mask_token_id, int32_t vocab,
                                  const void* const* k_ctx_layers,
                                  const void* const* v_ctx_layers, const int64_t* ctx_start,
                                  const int32_t* ctx_len, int32_t max_ctx_len, const void* ada_w,
                                  const float* ada_bias, const float* ada_table,
                                  const tt_step_provider* provider, int32_t* tokens,
                                  uint8_t* masked, int8_t* commit_step, int32_t* steps_taken,
                                  void* workspace, size_t workspace_bytes, tt_stream stream) {
  return denoise_common("tt_denoise_block_resume", shape, n_layers, first_step, max_steps, gamma,
                        temperature, sample, seed, block_index, mask_token_id, vocab,
                        k_ctx_layers, v_ctx_layers, ctx_start, ctx_len, max_ctx_len, ada_w,
                        ada_bias, ada_table, provider, tokens, masked, commit_step, steps_taken,
                        workspace, workspace_bytes, stream);
}

size_t tt_generate_workspace_size(const tt_attn_shape* shape, int32_t n_layers, int32_t n_blocks,
                                  int32_t max_ctx_len, int32_t vocab) {
  if (check_shape(shape) != TT_OK) return 0;
  if (n_layers < 1 || n_blocks < 0 || max_ctx_len < 0 || vocab < 1) {
    fail(TT_ERR_INVALID_ARG, "n_layers %d, n_blocks %d, max_ctx_len %d, vocab %d", n_layers,
         n_blocks, max_ctx_len, vocab);
    return 0;
  }
  ok();
  return generate_bytes(shape, n_layers, n_blocks, max_ctx_len, vocab);
}

tt_status tt_generate(const tt_attn_shape* shape, int32_t n_layers, int32_t n_blocks,
                      int32_t steps_per_block, float gamma, float temperature, int32_t sample,
                      uint64_t seed, int32_t mask_token_id, int32_t eos_token_id, int32_t vocab,
                      void* const* k_ctx_layers, void* const* v_ctx_layers,
                      const int64_t* ctx_start, const int64_t* ctx_end, int32_t* ctx_len,
                      int32_t max_ctx_len, const void* ada_w, const float* ada_bias,
                      const float* ada_table, const tt_gen_provider* provider,
                      int32_t* out_tokens, int32_t* n_generated, int8_t* stop_reason,
                      int32_t* blocks_taken, void* workspace, size_t workspace_bytes,
                      tt_stream stream) {
  const char* fn = "tt_generate";
  if (blocks_taken) *blocks_taken = 0;
  tt_status st = check_shape(shape);
  if (st != TT_OK) return st;
  const int B = shape->batch, S = shape->block_size;
  if (n_layers < 1) return fail(TT_ERR_INVALID_ARG, "%s: n_layers %d < 1", fn, n_layers);
  if (n_blocks < 0) return fail(TT_ERR_INVALID_ARG, "%s: n_blocks %d < 0", fn, n_blocks);
  if (steps_per_block < 1 || steps_per_block > S)
    return fail(TT_ERR_INVALID_ARG, "%s: steps_per_block %d outside [1, block_size=%d]", fn,
                steps_per_block, S);
  if (max_ctx_len < 0) return fail(TT_ERR_INVALID_ARG, "%s: max_ctx_len %d < 0", fn, max_ctx_len);
  if (static_cast<int64_t>(max_ctx_len) + static_cast<int64_t>(n_blocks) * S > INT32_MAX)
    return fail(TT_ERR_INVALID_ARG, "%s: max_ctx_len + n_blocks * S overflows int32", fn);
  st = check_unmask_scalars(B, S, vocab, vocab, gamma, temperature);
  if (st != TT_OK) return st;
  st = check_layers(fn, n_layers, const_cast<const void* const*>(k_ctx_layers),
                    const_cast<const void* const*>(v_ctx_layers));
  if (st != TT_OK) return st;
  if (!ctx_start || !ctx_end || !ctx_len)
    return fail(TT_ERR_INVALID_ARG, "%s: ctx_start, ctx_end and ctx_len must be non-NULL", fn);
  if (!aligned(ctx_start, 8) || !aligned(ctx_end, 8) || !aligned(ctx_len, 4))
    return fail(TT_ERR_INVALID_ARG, "%s: misaligned ctx_start/ctx_end/ctx_len", fn);
  if (!provider || !provider->layer_inputs || !provider->logits || !provider->ctx_inputs)
    return fail(TT_ERR_INVALID_ARG, "%s: provider and its three callbacks must be non-NULL", fn);
  if (!out_tokens || !n_generated)
    return fail(TT_ERR_INVALID_ARG, "%s: out_tokens and n_generated must be non-NULL", fn);
  if (!aligned(out_tokens, 4) || !aligned(n_generated, 4))
    return fail(TT_ERR_INVALID_ARG, "%s: misaligned out_tokens/n_generated", fn);
  st = check_ada(fn, shape, ada_w, ada_bias, ada_table);
  if (st != TT_OK) return st;
  if (B == 0) return ok();
  const size_t need = generate_bytes(shape, n_layers, n_blocks, max_ctx_len, vocab);
  if (!workspace || workspace_bytes < need)
    return fail(TT_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(TT_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);

  st = check_ctx_on_device(fn, B, ctx_start, ctx_len, ctx_end, nullptr, stream);
  if (st != TT_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int hint = max_ctx_len + n_blocks * S;
  Carver cv{static_cast<char*>(workspace)};
  const DenoiseBufs z = carve_denoise(cv, shape, n_layers, hint, vocab);
  int32_t* tokens = static_cast<int32_t*>(cv.take(static_cast<size_t>(B) * S * 4));
  uint8_t* masked = static_cast<uint8_t*>(cv.take(static_cast<size_t>(B) * S));
  uint8_t* unfinished = static_cast<uint8_t*>(cv.take(B));
  uint8_t* appended = static_cast<uint8_t*>(cv.take(B));
  hipError_t he = tt::launch_gen_init(B, unfinished, n_generated, stop_reason, hs);
  if (he != hipSuccess) return hip_fail(he, fn);
  LoopOpts o{};
  o.n_layers = n_layers; o.max_steps = steps_per_block; o.vocab = vocab;
  o.mask_id = mask_token_id; o.gamma = gamma; o.temperature = temperature;
  o.sample = sample != 0; o.seed = seed; o.finish_block = 1;
  for (int blk = 0; blk < n_blocks; ++blk) {
    // a fully masked block for every unfinished sequence; stop when none is left
    he = tt::launch_gen_block_init(B, S, mask_token_id, unfinished, tokens, masked, z.total, hs);
    int32_t host_left = 0;
    if (he == hipSuccess)
      he = hipMemcpyAsync(&host_left, z.total, sizeof(int32_t), hipMemcpyDeviceToHost, hs);
    if (he == hipSuccess) he = hipStreamSynchronize(hs);
    if (he != hipSuccess) return hip_fail(he, fn);
    if (host_left == 0) break;
    o.block = blk;
    auto layer_inputs = [&](int k, int l, const void* prev) {
      return provider->layer_inputs(provider->user, blk, k, l, prev, z.q, z.kb, z.vb, stream);
    };
    auto logits_fn = [&](int k) {
      return provider->logits(provider->user, blk, k, z.out, z.logits, stream);
    };
    st = denoise_loop(fn, shape, o, const_cast<const void* const*>(k_ctx_layers),
                      const_cast<const void* const*>(v_ctx_layers), ctx_start, ctx_len, ada_w,
                      ada_bias, ada_table, layer_inputs, logits_fn, tokens, masked, nullptr,
                      nullptr, z, stream);
    if (st != TT_OK) return st;
    // the context tower takes the block: every layer's causal attention with
    // the append of the block's K/V, then the lengths grow
    for (int l = 0; l < n_layers; ++l) {
      const int rc = provider->ctx_inputs(provider->user, blk, l, tokens, l == 0 ? nullptr : z.out,
                                          z.q, z.kb, z.vb, stream);
      if (rc != 0)
        return fail(TT_ERR_CALLBACK, "%s: ctx_inputs(block %d, layer %d) returned %d", fn, blk, l, rc);
      tt::AttnArgs a{};
      a.B = B; a.S = S; a.Hq = shape->n_q_heads; a.Hkv = shape->n_kv_heads; a.d = shape->head_dim;
      a.dtype = shape->dtype;
      a.q = z.q; a.kb = z.kb; a.vb = z.vb; a.kc = k_ctx_layers[l]; a.vc = v_ctx_layers[l];
      a.ctx_start = ctx_start; a.ctx_len = ctx_len; a.active = unfinished;
      a.out = z.out;
      a.causal = 1; a.ctx_end = ctx_end; a.kc_out = k_ctx_layers[l]; a.vc_out = v_ctx_layers[l];
      he = tt::launch_block_attn(a, z.ap, z.attn_ws, hs);
      if (he != hipSuccess) return hip_fail(he, fn);
    }
    he = tt::launch_ctx_advance(B, S, ctx_start, ctx_end, ctx_len, unfinished, appended, hs);
    if (he == hipSuccess)
      he = tt::launch_gen_block_commit(B, S, blk, n_blocks, eos_token_id, tokens, appended,
                                       unfinished, out_tokens, n_generated, stop_reason, hs);
    if (he != hipSuccess) return hip_fail(he, fn);
    if (blocks_taken) *blocks_taken = blk + 1;
  }
  he = hipStreamSynchronize(hs);
  if (he != hipSuccess) return hip_fail(he, "tt_generate final sync");
  return ok();
}

}  // extern "C"

// ------------------------------------------------- weighted adaLN sublayer

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + nb && y < x + na;
}

tt_status check_sublayer(const char* fn, const tt_attn_shape* s, int32_t width) {
  tt_status st = check_shape(s);
  if (st != TT_OK) return st;
  if (s->dtype != TT_BF16)
    return fail(TT_ERR_UNSUPPORTED, "%s: the weighted sublayer runs on bf16 storage only", fn);
  if (width < 64 || width % 64 != 0 || !tt::ln_supported(width))
    return fail(TT_ERR_UNSUPPORTED, "%s: width %d not supported (a multiple of 64, at most 8192)",
                fn, width);
  const int64_t M = static_cast<int64_t>(s->batch) * s->block_size;
  if (M > (int64_t(1) << 24)) return fail(TT_ERR_INVALID_ARG, "%s: batch * block_size too large", fn);
  const int nq = s->n_q_heads * s->head_dim, nk = s->n_kv_heads * s->head_dim;
  if (M > 0 && (!tt::gemm_supported(static_cast<int>(M), nq + 2 * nk, width) ||
                !tt::gemm_supported(static_cast<int>(M), width, nq)))
    return fail(TT_ERR_UNSUPPORTED, "%s: projection sizes not supported", fn);
  return TT_OK;
}

struct SubBufs {
  uint16_t *h, *q, *k, *v, *o;
  void* attn_ws;
};

size_t sublayer_bytes(const tt_attn_shape* s, int32_t width, int32_t max_ctx_len,
                      SubBufs* bufs, void* base) {
  const size_t M = static_cast<size_t>(s->batch) * s->block_size;
  const size_t nq = static_cast<size_t>(s->n_q_heads) * s->head_dim;
  const size_t nk = static_cast<size_t>(s->n_kv_heads) * s->head_dim;
  Carver c{static_cast<char*>(base)};
  void* h = c.take(M * width * 2);
  void* q = c.take(M * nq * 2);
  void* k = c.take(M * nk * 2);
  void* v = c.take(M * nk * 2);
  void* o = c.take(M * nq * 2);
  const tt::AttnPlan ap = tt::attn_plan(s->batch, s->block_size, s->n_q_heads, s->n_kv_heads,
                                        s->head_dim, s->dtype, max_ctx_len);
  void* w = c.take(ap.total_bytes);
  if (bufs) {
    bufs->h = static_cast<uint16_t*>(h); bufs->q = static_cast<uint16_t*>(q);
    bufs->k = static_cast<uint16_t*>(k); bufs->v = static_cast<uint16_t*>(v);
    bufs->o = static_cast<uint16_t*>(o); bufs->attn_ws = w;
  }
  return c.off;
}

tt::GemmArgs qkv_args(const tt_attn_shape* s, int32_t width, const void* h, const void* w_qkv,
                      const uint8_t* active, void* q, void* k, void* v) {
  tt::GemmArgs g{};
  g.M = s->batch * s->block_size; g.K = width; g.S = s->block_size;
  g.nq = s->n_q_heads * s->head_dim; g.nk = s->n_kv_heads * s->head_dim;
  g.N = g.nq + 2 * g.nk;
  g.a = static_cast<const uint16_t*>(h); g.w = static_cast<const uint16_t*>(w_qkv);
  g.active = active;
  g.q = static_cast<uint16_t*>(q); g.k = static_cast<uint16_t*>(k); g.v = static_cast<uint16_t*>(v);
  return g;
}

tt::GemmArgs out_args(const tt_attn_shape* s, int32_t width, const void* o, const void* w_o,
                      const float* gate, const void* x, const uint8_t* active, void* out) {
  tt::GemmArgs g{};
  g.M = s->batch * s->block_size; g.N = width; g.S = s->block_size;
  g.K = s->n_q_heads * s->head_dim;
  g.a = static_cast<const uint16_t*>(o); g.w = static_cast<const uint16_t*>(w_o);
  g.active = active;
  g.x = static_cast<const uint16_t*>(x); g.gate = gate; g.out = static_cast<uint16_t*>(out);
  return g;
}

}  // namespace

extern "C" {

tt_status tt_ln_modulate(const tt_attn_shape* shape, int32_t width, const void* x,
                         const float* shift, const float* scale, const uint8_t* active, void* h,
                         tt_stream stream) {
  const char* fn = "tt_ln_modulate";
  tt_status st = check_sublayer(fn, shape, width);
  if (st != TT_OK) return st;
  if (!x || !shift || !scale || !h)
    return fail(TT_ERR_INVALID_ARG, "%s: x, shift, scale and h must be non-NULL", fn);
  const void* ptrs[] = {x, shift, scale, h};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(TT_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  const size_t M = static_cast<size_t>(shape->batch) * shape->block_size;
  if (x != h && overlaps(x, M * width * 2, h, M * width * 2))
    return fail(TT_ERR_INVALID_ARG, "%s: h overlaps x without being x", fn);
  if (M == 0) return ok();
  tt::LnArgs a{};
  a.M = static_cast<int>(M); a.S = shape->block_size; a.D = width;
  a.x = static_cast<const uint16_t*>(x); a.shift = shift; a.scale = scale; a.active = active;
  a.h = static_cast<uint16_t*>(h);
  const hipError_t e = tt::launch_ln_modulate(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

tt_status tt_qkv_proj(const tt_attn_shape* shape, int32_t width, const void* h, const void* w_qkv,
                      const uint8_t* active, void* q_blk, void* k_blk, void* v_blk,
                      tt_stream stream) {
  const char* fn = "tt_qkv_proj";
  tt_status st = check_sublayer(fn, shape, width);
  if (st != TT_OK) return st;
  if (!h || !w_qkv || !q_blk || !k_blk || !v_blk)
    return fail(TT_ERR_INVALID_ARG, "%s: h, w_qkv, q_blk, k_blk and v_blk must be non-NULL", fn);
  const void* ptrs[] = {h, w_qkv, q_blk, k_blk, v_blk};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(TT_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  const size_t M = static_cast<size_t>(shape->batch) * shape->block_size;
  const size_t nq = static_cast<size_t>(shape->n_q_heads) * shape->head_dim;
  const size_t nk = static_cast<size_t>(shape->n_kv_heads) * shape->head_dim;
  if (overlaps(h, M * width * 2, q_blk, M * nq * 2) || overlaps(h, M * width * 2, k_blk, M * nk * 2) ||
      overlaps(h, M * width * 2, v_blk, M * nk * 2))
    return fail(TT_ERR_INVALID_ARG, "%s: q/k/v overlap h", fn);
  if (M == 0) return ok();
  const tt::GemmArgs g = qkv_args(shape, width, h, w_qkv, active, q_blk, k_blk, v_blk);
  const hipError_t e = tt::launch_gemm(g, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

tt_status tt_out_proj(const tt_attn_shape* shape, int32_t width, const void* o, const void* w_o,
                      const float* gate, const void* x, const uint8_t* active, void* out,
                      tt_stream stream) {
  const char* fn = "tt_out_proj";
  tt_status st = check_sublayer(fn, shape, width);
  if (st != TT_OK) return st;
  if (!o || !w_o || !gate || !x || !out)
    return fail(TT_ERR_INVALID_ARG, "%s: o, w_o, gate, x and out must be non-NULL", fn);
  const void* ptrs[] = {o, w_o, gate, x, out};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(TT_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  const size_t M = static_cast<size_t>(shape->batch) * shape->block_size;
  const size_t nq = static_cast<size_t>(shape->n_q_heads) * shape->head_dim;
  if (overlaps(o, M * nq * 2, out, M * width * 2) ||
      (x != out && overlaps(x, M * width * 2, out, M * width * 2)))
    return fail(TT_ERR_INVALID_ARG, "%s: out overlaps o, or overlaps x without being x", fn);
  if (M == 0) return ok();
  const tt::GemmArgs g = out_args(shape, width, o, w_o, gate, x, active, out);
  const hipError_t e = tt::launch_gemm(g, 1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

size_t tt_adaln_sublayer_workspace_size(const tt_attn_shape* shape, int32_t width,
                                        int32_t max_ctx_len) {
  if (check_sublayer("tt_adaln_sublayer_workspace_size", shape, width) != TT_OK) return 0;
  if (max_ctx_len < 0) {
    fail(TT_ERR_INVALID_ARG, "max_ctx_len %d < 0", max_ctx_len);
    return 0;
  }
  ok();
  const size_t n = sublayer_bytes(shape, width, max_ctx_len, nullptr, nullptr);
  return n < 256 ? 256 : n;
}

tt_status tt_adaln_attn_sublayer(const tt_attn_shape* shape, int32_t width, const void* x,
                                 const float* shift, const float* scale, const float* gate,
                                 const void* w_qkv, const void* w_o, const void* k_ctx,
                                 const void* v_ctx, const int64_t* ctx_start,
                                 const int32_t* ctx_len, int32_t max_ctx_len,
                                 const uint8_t* active, void* out, void* workspace,
                                 size_t workspace_bytes, tt_stream stream) {
  const char* fn = "tt_adaln_attn_sublayer";
  tt_status st = check_sublayer(fn, shape, width);
  if (st != TT_OK) return st;
  if (max_ctx_len < 0) return fail(TT_ERR_INVALID_ARG, "%s: max_ctx_len %d < 0", fn, max_ctx_len);
  if (!x || !shift || !scale || !gate || !w_qkv || !w_o || !out)
    return fail(TT_ERR_INVALID_ARG, "%s: x, shift, scale, gate, w_qkv, w_o and out must be non-NULL", fn);
  if (!k_ctx || !v_ctx || !ctx_start || !ctx_len)
    return fail(TT_ERR_INVALID_ARG, "%s: k_ctx, v_ctx, ctx_start and ctx_len must be non-NULL", fn);
  const void* ptrs[] = {x, shift, scale, gate, w_qkv, w_o, k_ctx, v_ctx, out};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(TT_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  if (!aligned(ctx_start, 8) || !aligned(ctx_len, 4))
    return fail(TT_ERR_INVALID_ARG, "%s: misaligned ctx_start/ctx_len", fn);
  const size_t M = static_cast<size_t>(shape->batch) * shape->block_size;
  if (x != out && overlaps(x, M * width * 2, out, M * width * 2))
    return fail(TT_ERR_INVALID_ARG, "%s: out overlaps x without being x", fn);
  if (M == 0) return ok();
  const size_t need = sublayer_bytes(shape, width, max_ctx_len, nullptr, nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(TT_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, workspace_bytes, need);
  if (!aligned(workspace, 256))
    return fail(TT_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  st = check_ctx_on_device(fn, shape->batch, ctx_start, ctx_len, nullptr, active, stream);
  if (st != TT_OK) return st;
  SubBufs w{};
  sublayer_bytes(shape, width, max_ctx_len, &w, workspace);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  tt::LnArgs la{};
  la.M = static_cast<int>(M); la.S = shape->block_size; la.D = width;
  la.x = static_cast<const uint16_t*>(x); la.shift = shift; la.scale = scale; la.active = active;
  la.h = w.h;
  hipError_t e = tt::launch_ln_modulate(la, hs);
  if (e == hipSuccess)
    e = tt::launch_gemm(qkv_args(shape, width, w.h, w_qkv, active, w.q, w.k, w.v), 0, hs);
  if (e == hipSuccess) {
    tt::AttnArgs a{};
    a.B = shape->batch; a.S = shape->block_size; a.Hq = shape->n_q_heads;
    a.Hkv = shape->n_kv_heads; a.d = shape->head_dim; a.dtype = shape->dtype;
    a.q = w.q; a.kb = w.k; a.vb = w.v; a.kc = k_ctx; a.vc = v_ctx;
    a.ctx_start = ctx_start; a.ctx_len = ctx_len; a.active = active;
    a.out = w.o;
    a.kc_out = const_cast<void*>(k_ctx);
    a.vc_out = const_cast<void*>(v_ctx);
    const tt::AttnPlan p = tt::attn_plan(shape->batch, shape->block_size, shape->n_q_heads,
                                         shape->n_kv_heads, shape->head_dim, shape->dtype,
                                         max_ctx_len);
    e = tt::launch_block_attn(a, p, w.attn_ws, hs);
  }
  if (e == hipSuccess)
    e = tt::launch_gemm(out_args(shape, width, w.o, w_o, gate, x, active, out), 1, hs);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // extern "C"
