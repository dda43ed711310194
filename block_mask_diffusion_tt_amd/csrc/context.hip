// The context tower's bookkeeping after it has consumed a committed block:
// every context with room grows by the S block tokens whose K/V the
// context-tower attention call has just written after it ([dothoosh]
// two-tower mechanism section: the context tower runs causally over the
// prompt and the committed tokens and keeps every layer's KV cache); and the
// generation loop's per-block state ([dothoosh] two-tower mechanism section:
// generation goes block by block, each block starting as [MASK] tokens;
// [news] training and inference section, code example: the generation call
// takes max_new_tokens, block_size and eos_token_id).
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

// Generation state: every sequence unfinished, nothing generated yet.
__global__ void gen_init_kernel(int B, uint8_t* unfinished, int32_t* n_generated, int8_t* stop) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  unfinished[b] = 1;
  n_generated[b] = 0;
  if (stop) stop[b] = 0;
}

// A fully masked block for every unfinished sequence (finished ones get no
// masked slot, so the denoising loop leaves them inactive), and the number
// of unfinished sequences.  One workgroup.
__global__ void gen_block_init_kernel(int B, int S, int mask_id, const uint8_t* unfinished,
                                      int32_t* tokens, uint8_t* masked, int32_t* n_unfinished) {
  int local = 0;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int u = unfinished[b] != 0;
    local += u;
    for (int s = 0; s < S; ++s) {
      tokens[static_cast<int64_t>(b) * S + s] = mask_id;
      masked[static_cast<int64_t>(b) * S + s] = static_cast<uint8_t>(u);
    }
  }
  for (int off = 32; off >= 1; off >>= 1) local += __shfl_xor(local, off);
  __shared__ int part[16];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) t += part[w];
    *n_unfinished = t;
  }
}

// After the context tower took the block: the unfinished sequences' tokens
// go to out_tokens[b, block*S ..]; a sequence stops when the block holds EOS
// (stop 1) or its cache had no room for the block (stop 2).  One thread per
// sequence.
__global__ void gen_block_commit_kernel(int B, int S, int block, int n_blocks, int eos_id,
                                        const int32_t* tokens, const uint8_t* appended,
                                        uint8_t* unfinished, int32_t* out_tokens,
                                        int32_t* n_generated, int8_t* stop) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B || !unfinished[b]) return;
  const int64_t row = static_cast<int64_t>(b) * n_blocks * S + static_cast<int64_t>(block) * S;
  int eos = 0;
  for (int s = 0; s < S; ++s) {
    const int32_t t = tokens[static_cast<int64_t>(b) * S + s];
    out_tokens[row + s] = t;
    eos |= (eos_id >= 0 && t == eos_id);
  }
  n_generated[b] += S;
  if (eos || !appended[b]) {
    unfinished[b] = 0;
    if (stop) stop[b] = static_cast<int8_t>(eos ? 1 : 2);
  }
}

}  // namespace

hipError_t launch_gen_init(int B, uint8_t* unfinished, int32_t* n_generated, int8_t* stop,
                           hipStream_t st) {
  hipLaunchKernelGGL(gen_init_kernel, dim3(static_cast<unsigned>(ceil_div(B, 256))), dim3(256), 0, st,
                     B, unfinished, n_generated, stop);
  return hipGetLastError();
}

hipError_t launch_gen_block_init(int B, int S, int mask_id, const uint8_t* unfinished,
                                 int32_t* tokens, uint8_t* masked, int32_t* n_unfinished,
                                 hipStream_t st) {
  hipLaunchKernelGGL(gen_block_init_kernel, dim3(1), dim3(1024), 0, st, B, S, mask_id, unfinished,
                     tokens, masked, n_unfinished);
  return hipGetLastError();
}

hipError_t launch_gen_block_commit(int B, int S, int block, int n_blocks, int eos_id,
                                   const int32_t* tokens, const uint8_t* appended,
                                   uint8_t* unfinished, int32_t* out_tokens,
                                   int32_t* n_generated, int8_t* stop, hipStream_t st) {
  hipLaunchKernelGGL(gen_block_commit_kernel, dim3(static_cast<unsigned>(ceil_div(B, 256))), dim3(256),
                     0, st, B, S, block, n_blocks, eos_id, tokens, appended, unfinished, out_tokens,
                     n_generated, stop);
  return hipGetLastError();
}

hipError_t launch_ctx_advance(int B, int S, const int64_t* ctx_start, const int64_t* ctx_end,
                              int32_t* ctx_len, const uint8_t* active, uint8_t* appended,
                              hipStream_t st) {
  hipLaunchKernelGGL(ctx_advance_kernel, dim3(static_cast<unsigned>(ceil_div(B, 256))), dim3(256), 0,
                     st, B, S, ctx_start, ctx_end, ctx_len, active, appended);
  return hipGetLastError();
}

}  // namespace tt
