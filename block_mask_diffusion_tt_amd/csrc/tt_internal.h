// Internal declarations shared by the libtt translation units: launch
// parameter blocks, sizing rules and the kernel launchers.  Nothing here is
// part of the C ABI (include/tt.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tt {

// Compute units of the current device (asked once per device); the MI355X's
// 256 when no device can be asked (a workspace size computed on a host
// without a GPU).  Launch plans, and so workspace sizes, follow the device
// that is current when they are computed.
int device_cus();

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- attention
// Rows of one (sequence, KV head) group: r = s * G + j  (block slot s, query
// head h = g * G + j).  Keys of a unit: the block's S keys (chunk 0 only)
// then context tokens [c * chunk, end).  Partials of unit u = (((b * Hkv + g)
// * RB + rb) * NC + c) hold, per row of the row block, (m, l, k, 0) in fp32
// -- the running max m (log2 units), the sum l and a scale exponent k --
// and the normalised output o = acc / l times 2^-k: d fp16 values for bf16
// storage (k keeps |o 2^-k| below 2^15), d fp32 values with k = 0 for fp32.
struct AttnPlan {
  int64_t groups;     // B * Hkv * RB
  int rows;           // R = S * G
  int rows_per_unit;  // rows a workgroup owns (row block height)
  int row_blocks;     // RB
  int chunk;          // context keys per unit (multiple of 64)
  int n_chunks;       // NC: unit slots per (b, g, rb)
  size_t part_acc_bytes;
  size_t part_ml_bytes;
  size_t total_bytes;
};

struct AttnArgs {
  int B, S, Hq, Hkv, d, dtype;
  const void* q; const void* kb; const void* vb;
  const void* kc; const void* vc;
  const int64_t* ctx_start; const int32_t* ctx_len;
  const uint8_t* active;
  const float* shift; const float* scale; const float* gate;
  const void* residual; void* out; float* lse;
  // Context-tower form: causal inside the block (slot s sees block keys
  // 0..s), and, when ctx_end is set, the block's K/V written into the cache
  // rows right after each sequence's context (kc_out/vc_out alias kc/vc).
  int causal;
  const int64_t* ctx_end; void* kc_out; void* vc_out;
};

AttnPlan attn_plan(int B, int S, int Hq, int Hkv, int d, int dtype, int max_ctx_len);
hipError_t launch_block_attn(const AttnArgs& a, const AttnPlan& p, void* ws, hipStream_t st);

// ---------------------------------------------------------------- unmasking
struct UnmaskPlan {
  int splits;      // workgroups per row (argmax pass)
  int split_len;   // vocab entries per split (multiple of 8)
  int s_splits;    // workgroups per row (sampling pass: fixed slices)
  size_t part_bytes;
  size_t s_part_bytes;
  size_t total_bytes;  // enough for either pass
};

struct UnmaskArgs {
  int B, S, V, dtype;
  const void* logits; int64_t row_stride;
  float gamma, temperature;
  int mask_id, step;
  int32_t* tokens; uint8_t* masked;
  uint8_t* committed_now; float* conf; int32_t* pred;
  int8_t* commit_step; int32_t* n_masked;
  // temperature sampling (Gumbel-max over Philox4x32-10 noise) when set
  int sample; uint64_t seed; int block_index;
};

UnmaskPlan unmask_plan(int B, int S, int V);
hipError_t launch_confidence_unmask(const UnmaskArgs& a, const UnmaskPlan& p, void* ws,
                                    hipStream_t st);

// ---------------------------------------------------------------- Mamba-2
// One layer's mixer over a block, seeded with the context's states
// (csrc/mamba.hip).  Channels of xbc: x (H*P), then B (G*N), then C (G*N).
struct MambaArgs {
  int B, S, H, P, N, G, W, dtype;
  const void* xbc; const float* dt_raw;
  const void* conv_state; const float* ssm_state;
  const float* conv_w; const float* conv_b; const float* A_log; const float* dt_bias;
  const float* D; const uint8_t* active;
  void* y; void* conv_state_out; float* ssm_state_out;
};

bool mamba_supported(int P, int N, int W);
// whether one launch does the whole layer (no group kernel, workspace unused)
bool mamba_fused(int S, int P, int N);
size_t mamba_lds_bytes(int S, int P, int N);
size_t mamba_group_lds_bytes(int S, int N);
size_t mamba_workspace_bytes(int B, int S, int G, int N);
hipError_t launch_mamba_scan(const MambaArgs& a, void* ws, hipStream_t st);

// ------------------------------------------------- weighted adaLN sublayer
// LayerNorm (no affine, eps 1e-6) + modulation of M = B*S token rows of
// width D (bf16 in and out; shift/scale fp32 [B, D]).
struct LnArgs {
  int M, S, D;
  const uint16_t* x; const float* shift; const float* scale; const uint8_t* active;
  uint16_t* h;
};
bool ln_supported(int D);
hipError_t launch_ln_modulate(const LnArgs& a, hipStream_t st);

// C[M, N] = A[M, K] W[N, K]^T (bf16, fp32 accumulation) with an epilogue:
// epi 0 scatters columns [0, nq) / [nq, nq+nk) / [nq+nk, N) to q [M, nq],
// k [M, nk], v [M, nk]; epi 1 writes out = x + gate[m / S] * C ([M, N]).
// Rows of inactive sequences are not written.
struct GemmArgs {
  int M, N, K, S;
  const uint16_t* a; const uint16_t* w; const uint8_t* active;
  int nq, nk; uint16_t* q; uint16_t* k; uint16_t* v;
  const uint16_t* x; const float* gate; uint16_t* out;
};
bool gemm_supported(int M, int N, int K);
hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st);

// ---------------------------------------------------------------- adaLN
hipError_t launch_timestep_embed(int B, const float* t, const int32_t* n_masked, int S,
                                 float* emb, hipStream_t st);
hipError_t launch_adaln_single(int B, int width, int n_layers, const float* emb,
                               const void* w, const float* bias, const float* table,
                               float* ada, hipStream_t st);
hipError_t launch_active_from_masked(int B, const int32_t* n_masked, uint8_t* active,
                                     int32_t* total, hipStream_t st);
hipError_t launch_count_masked(int B, int S, const uint8_t* masked, int32_t* n_masked,
                               hipStream_t st);
hipError_t launch_clear(void* p, size_t bytes, hipStream_t st);
// Generation bookkeeping (csrc/context.hip).
hipError_t launch_gen_init(int B, uint8_t* unfinished, int32_t* n_generated, int8_t* stop,
                           hipStream_t st);
hipError_t launch_gen_block_init(int B, int S, int mask_id, const uint8_t* unfinished,
                                 int32_t* tokens, uint8_t* masked, int32_t* n_unfinished,
                                 hipStream_t st);
hipError_t launch_gen_block_commit(int B, int S, int block, int n_blocks, int eos_id,
                                   const int32_t* tokens, const uint8_t* appended,
                                   uint8_t* unfinished, int32_t* out_tokens,
                                   int32_t* n_generated, int8_t* stop, hipStream_t st);
hipError_t launch_ctx_advance(int B, int S, const int64_t* ctx_start, const int64_t* ctx_end,
                              int32_t* ctx_len, const uint8_t* active, uint8_t* appended,
                              hipStream_t st);

// ---------------------------------------------------------------- TT_VALIDATE
// Checks the context arrays on the device (csrc/validate.hip) and waits for
// the outcome: outcome[0] = the first failing sequence or -1, outcome[1] the
// rule (1 ctx_len < 0, 2 ctx_start < 0, 3 ctx_end below start + len, 4 two
// reserved regions overlap, outcome[2] = the other sequence), outcome[2..3]
// the values involved.
hipError_t validate_ctx(int B, const int64_t* ctx_start, const int32_t* ctx_len,
                        const int64_t* ctx_end, const uint8_t* active, int64_t outcome[4],
                        hipStream_t st);

}  // namespace tt
