// Mamba-2 sequence mixer of one layer over a block of S slots, seeded with
// the context tower's conv/SSM boundary state.
//
// [dothoosh] two-tower mechanism section: the context tower produces every
// layer's KV cache and final Mamba-2 states, and the denoiser's Mamba-2
// layers take their initial state directly from the context tower's Mamba
// state.  [modelcard] notes: the seeding injects the context tower's conv and
// SSM boundary states as the initial states of the denoiser's Mamba layers,
// causally.  The mixer is the published Mamba-2 one (Dao & Gu, ICML 2024):
// depthwise causal conv of width W over (x, B, C), SiLU, then per head the
// scalar-decay selective scan H_s = exp(dt_s A) H_{s-1} + dt_s x_s B_s^T,
// y_s = H_s C_s + D x_s, dt_s = softplus(dt_raw_s + dt_bias).
//
// One workgroup per (sequence b, head h), 256 threads, HBM-bound on the
// fp32 SSM state (P x N floats per head: 32 KB at P = 64, N = 128):
//   1. conv: thread c walks channel c of the head's x channels and its
//      group's B and C channels down the S slots with a sliding window that
//      starts from the conv state (every input read once), writing SiLU
//      outputs to LDS as [S][P + 2N] fp32; S threads write dt_s and the
//      decay a_s to LDS;
//   2. scan: thread (p, q) holds H[p][q*NPT .. q*NPT+NPT) in registers
//      (NPT = N / (256 / P)), loaded with 16-byte loads; per slot it updates
//      them with a_s and dt_s x_s[p] B_s and forms its partial of H_s C_s;
//      the 256/P threads of a row reduce by shuffles; y goes through LDS and
//      leaves as coalesced rows;
//   3. optionally (the context tower taking a committed block) the final
//      state is written back (in place allowed: every thread reads its part
//      before anyone writes) and the conv state becomes the block's last
//      W-1 inputs (to a separate buffer: the B/C channels are read by every
//      head of the group).
#include <math.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kMThreads = 256;
constexpr int kMaxConvW = 8;

__device__ __forceinline__ float ld_elt(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float ld_elt(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void st_elt(uint16_t* p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}
__device__ __forceinline__ void st_elt(float* p, int64_t i, float v) { p[i] = v; }

__device__ __forceinline__ float silu(float v) { return v / (1.f + __expf(-v)); }
__device__ __forceinline__ float softplus(float v) { return v > 20.f ? v : log1pf(expf(v)); }

template <typename T, int P, int N>
__global__ __launch_bounds__(kMThreads) void mamba_scan_kernel(MambaArgs a) {
  constexpr int TPR = kMThreads / P;     // threads per state row
  constexpr int NPT = N / TPR;           // state entries per thread
  static_assert(NPT % 4 == 0, "16-byte state loads");
  const int b = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  if (a.active && !a.active[b]) return;
  const int tid = threadIdx.x;
  const int S = a.S, W = a.W, H = a.H, G = a.G;
  const int g = h / (H / G);
  const int C = H * P + 2 * G * N;
  const int CH = P + 2 * N;              // this head's channels: x, then B, C of its group
  extern __shared__ float lds[];
  float* conv_out = lds;                 // [S][CH]
  float* s_dt = lds + S * CH;            // [S]
  float* s_a = s_dt + S;                 // [S]
  float* s_y = s_a + S;                  // [S][P]
  const T* xbc = static_cast<const T*>(a.xbc) + static_cast<int64_t>(b) * S * C;
  const T* cst = static_cast<const T*>(a.conv_state) + static_cast<int64_t>(b) * C * (W - 1);

  // ---- state loads first (the HBM-heavy part), then the convolution
  const int p = tid / TPR, q = tid % TPR;
  const int64_t sbase = ((static_cast<int64_t>(b) * H + h) * P + p) * N + q * NPT;
  float st[NPT];
#pragma unroll
  for (int j = 0; j < NPT; j += 4) {
    const float4 v = *reinterpret_cast<const float4*>(a.ssm_state + sbase + j);
    st[j] = v.x; st[j + 1] = v.y; st[j + 2] = v.z; st[j + 3] = v.w;
  }
  for (int cl = tid; cl < CH; cl += kMThreads) {
    const int c = cl < P ? h * P + cl
                         : (cl < P + N ? H * P + g * N + (cl - P) : H * P + G * N + g * N + (cl - P - N));
    // the W-1 previous inputs and the taps, in registers (fixed-size arrays
    // with predicated entries: W <= kMaxConvW)
    float win[kMaxConvW - 1], w[kMaxConvW];
#pragma unroll
    for (int j = 0; j < kMaxConvW - 1; ++j)
      win[j] = j < W - 1 ? ld_elt(cst, static_cast<int64_t>(c) * (W - 1) + j) : 0.f;
#pragma unroll
    for (int j = 0; j < kMaxConvW; ++j) w[j] = j < W ? a.conv_w[static_cast<int64_t>(c) * W + j] : 0.f;
    const float bias = a.conv_b ? a.conv_b[c] : 0.f;
    for (int s = 0; s < S; ++s) {
      const float cur = ld_elt(xbc, static_cast<int64_t>(s) * C + c);
      float acc = bias;
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j)
        if (j < W - 1) acc = fmaf(w[j], win[j], acc);
#pragma unroll
      for (int j = 0; j < kMaxConvW; ++j)
        if (j == W - 1) acc = fmaf(w[j], cur, acc);
      conv_out[s * CH + cl] = silu(acc);
#pragma unroll
      for (int j = 0; j < kMaxConvW - 1; ++j) {
        const float nxt = j + 1 < kMaxConvW - 1 ? win[j + 1] : 0.f;
        if (j < W - 2) win[j] = nxt;
        else if (j == W - 2) win[j] = cur;
      }
    }
  }
  if (tid < S) {
    const float A = -expf(a.A_log[h]);
    const float dt = softplus(a.dt_raw[(static_cast<int64_t>(b) * S + tid) * H + h] +
                              (a.dt_bias ? a.dt_bias[h] : 0.f));
    s_dt[tid] = dt;
    s_a[tid] = expf(dt * A);
  }
  __syncthreads();

  // ---- the scan
  const float Dh = a.D ? a.D[h] : 0.f;
  const float* Bs = conv_out + P + q * NPT;
  const float* Cs = conv_out + P + N + q * NPT;
  for (int s = 0; s < S; ++s) {
    const float as = s_a[s];
    const float x = conv_out[s * CH + p];
    const float dx = s_dt[s] * x;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NPT; j += 4) {
      const float4 bv = *reinterpret_cast<const float4*>(Bs + s * CH + j);
      const float4 cv = *reinterpret_cast<const float4*>(Cs + s * CH + j);
      st[j] = fmaf(as, st[j], dx * bv.x);
      st[j + 1] = fmaf(as, st[j + 1], dx * bv.y);
      st[j + 2] = fmaf(as, st[j + 2], dx * bv.z);
      st[j + 3] = fmaf(as, st[j + 3], dx * bv.w);
      acc = fmaf(st[j], cv.x, acc);
      acc = fmaf(st[j + 1], cv.y, acc);
      acc = fmaf(st[j + 2], cv.z, acc);
      acc = fmaf(st[j + 3], cv.w, acc);
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, TPR);
    if (q == 0) s_y[s * P + p] = acc + Dh * x;
  }
  __syncthreads();
  T* y = static_cast<T*>(a.y) + (static_cast<int64_t>(b) * S) * (H * P) + h * P;
  for (int i = tid; i < S * P; i += kMThreads)
    st_elt(y, static_cast<int64_t>(i / P) * (H * P) + i % P, s_y[i]);

  // ---- the context tower's state update
  if (a.ssm_state_out) {
#pragma unroll
    for (int j = 0; j < NPT; j += 4)
      *reinterpret_cast<float4*>(a.ssm_state_out + sbase + j) = make_float4(st[j], st[j + 1], st[j + 2], st[j + 3]);
  }
  if (a.conv_state_out) {
    T* cso = static_cast<T*>(a.conv_state_out) + static_cast<int64_t>(b) * C * (W - 1);
    // x channels by their head; B and C channels by the group's first head.
    // New state = the last W-1 of [old state ; block inputs].
    const bool owns_bc = (h % (H / G)) == 0;
    for (int cl = tid; cl < CH; cl += kMThreads) {
      if (cl >= P && !owns_bc) continue;
      const int c = cl < P ? h * P + cl
                           : (cl < P + N ? H * P + g * N + (cl - P) : H * P + G * N + g * N + (cl - P - N));
      for (int j = 0; j < W - 1; ++j) {
        const int t = S + j;             // position in [old state (W-1) ; block (S)]
        const float v = t < W - 1 ? ld_elt(cst, static_cast<int64_t>(c) * (W - 1) + t)
                                  : ld_elt(xbc, static_cast<int64_t>(t - (W - 1)) * C + c);
        st_elt(cso, static_cast<int64_t>(c) * (W - 1) + j, v);
      }
    }
  }
}

template <typename T>
hipError_t launch_t(const MambaArgs& a, hipStream_t st) {
  const size_t lds = mamba_lds_bytes(a.S, a.P, a.N);
  const dim3 grid(static_cast<unsigned>(a.B * a.H)), blk(kMThreads);
  // more than 64 KB of dynamic LDS must be allowed per kernel (up to 160 KB)
#define TT_MAMBA(PP, NN)                                                                   \
  if (a.P == PP && a.N == NN) {                                                            \
    if (lds > 65536) {                                                                     \
      const hipError_t e = hipFuncSetAttribute(                                            \
          reinterpret_cast<const void*>(&mamba_scan_kernel<T, PP, NN>),                    \
          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));              \
      if (e != hipSuccess) return e;                                                       \
    }                                                                                      \
    hipLaunchKernelGGL((mamba_scan_kernel<T, PP, NN>), grid, blk, lds, st, a);            \
    return hipGetLastError();                                                              \
  }
  TT_MAMBA(64, 128)
  TT_MAMBA(64, 64)
  TT_MAMBA(32, 128)
  TT_MAMBA(32, 64)
#undef TT_MAMBA
  return hipErrorInvalidValue;
}

}  // namespace

bool mamba_supported(int P, int N) {
  return (P == 64 || P == 32) && (N == 128 || N == 64);
}

size_t mamba_lds_bytes(int S, int P, int N) {
  return (static_cast<size_t>(S) * (P + 2 * N) + 2 * S + static_cast<size_t>(S) * P) * sizeof(float);
}

hipError_t launch_mamba_scan(const MambaArgs& a, hipStream_t st) {
  return a.dtype == 0 ? launch_t<uint16_t>(a, st) : launch_t<float>(a, st);
}

}  // namespace tt
