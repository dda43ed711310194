// The context tower's bookkeeping after it has consumed a committed block:
// every context with room grows by the S block tokens whose K/V the
// context-tower attention call has just written after it ([dothoosh]
// two-tower mechanism section: the context tower runs causally over the
// prompt and the committed tokens and keeps every layer's KV cache).
#include "tt_internal.h"

namespace tt {
namespace {

// One thread per sequence.  The room test is the one the attention call's
// append uses: ctx_len + S <= ctx_end - ctx_start.
__global__ void ctx_advance_kernel(int B, int S, const int64_t* ctx_start, const int64_t* ctx_end,
                                   int32_t* ctx_len, const uint8_t* active, uint8_t* appended) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int64_t L = ctx_len[b];
  const bool ok = (!active || active[b]) && L + S <= ctx_end[b] - ctx_start[b];
  if (ok) ctx_len[b] = static_cast<int32_t>(L + S);
  if (appended) appended[b] = ok ? 1 : 0;
}

}  // namespace

hipError_t launch_ctx_advance(int B, int S, const int64_t* ctx_start, const int64_t* ctx_end,
                              int32_t* ctx_len, const uint8_t* active, uint8_t* appended,
                              hipStream_t st) {
  hipLaunchKernelGGL(ctx_advance_kernel, dim3(static_cast<unsigned>(ceil_div(B, 256))), dim3(256), 0,
                     st, B, S, ctx_start, ctx_end, ctx_len, active, appended);
  return hipGetLastError();
}

}  // namespace tt
