// Device-side argument checks of the context arrays, run before a call's
// kernels when the environment sets TT_VALIDATE (a debugging aid: each
// checked call waits for the check's result, so calls become synchronous).
// The host can see every other argument; these arrays live on the device and
// decide which cache rows the kernels read and write.
#include <limits.h>

#include "tt_internal.h"

namespace tt {
namespace {

// The outcome of the last check on this device: the first failing sequence
// (-1 if none), the failed rule, two values for the message.  Only device
// code writes it; the host copies it out through the symbol.
__device__ int64_t g_outcome[4];

constexpr int kOverlapMaxB = 8192;   // pairwise region check up to this batch

// Rules, for sequence b with active[b] (or no active array):
//   1 ctx_len[b] < 0;  2 ctx_start[b] < 0;
//   3 ctx_end[b] < ctx_start[b] + ctx_len[b] (the context does not fit its
//     reserved region);
//   4 the reserved regions [ctx_start, ctx_end) of b and of another active
//     sequence overlap (v1 = that sequence).
__device__ int ctx_rule(int b, int B, const int64_t* ctx_start, const int32_t* ctx_len,
                        const int64_t* ctx_end, const uint8_t* active, int64_t& v1,
                        int64_t& v2) {
  const int64_t st = ctx_start[b];
  const int32_t L = ctx_len[b];
  if (L < 0) { v1 = L; v2 = 0; return 1; }
  if (st < 0) { v1 = st; v2 = 0; return 2; }
  if (!ctx_end) return 0;
  const int64_t en = ctx_end[b];
  if (en < st + L) { v1 = en; v2 = st + L; return 3; }
  if (B > kOverlapMaxB || en == st) return 0;
  for (int c = 0; c < B; ++c) {
    if (c == b || (active && !active[c])) continue;
    const int64_t s2 = ctx_start[c], e2 = ctx_end[c];
    if (s2 < e2 && s2 < en && st < e2) { v1 = c; v2 = 0; return 4; }
  }
  return 0;
}

__global__ __launch_bounds__(1024) void validate_ctx_kernel(int B, const int64_t* ctx_start,
                                                            const int32_t* ctx_len,
                                                            const int64_t* ctx_end,
                                                            const uint8_t* active) {
  __shared__ int first;
  if (threadIdx.x == 0) first = INT_MAX;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    if (active && !active[b]) continue;
    int64_t v1, v2;
    if (ctx_rule(b, B, ctx_start, ctx_len, ctx_end, active, v1, v2)) atomicMin(&first, b);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t v1 = 0, v2 = 0;
    int rule = 0;
    if (first != INT_MAX) rule = ctx_rule(first, B, ctx_start, ctx_len, ctx_end, active, v1, v2);
    g_outcome[0] = first == INT_MAX ? -1 : first;
    g_outcome[1] = rule;
    g_outcome[2] = v1;
    g_outcome[3] = v2;
  }
}

}  // namespace

hipError_t validate_ctx(int B, const int64_t* ctx_start, const int32_t* ctx_len,
                        const int64_t* ctx_end, const uint8_t* active, int64_t outcome[4],
                        hipStream_t st) {
  hipLaunchKernelGGL(validate_ctx_kernel, dim3(1), dim3(1024), 0, st, B, ctx_start, ctx_len,
                     ctx_end, active);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(outcome, HIP_SYMBOL(g_outcome), 4 * sizeof(int64_t), 0,
                               hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace tt
