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
// One workgroup per (sequence b, head h), 256 threads.  The block is short
// (S <= 64), so the scan is evaluated in its state-space-duality form (Dao &
// Gu): with cum_s = sum_{k<=s} dt_k A,
//   y_s = exp(cum_s) H0 C_s + sum_{j<=s} dt_j exp(cum_s - cum_j) (C_s . B_j) x_j
//         + D x_s
// which needs one multiply-add per state entry and slot (H0 C_s) instead of
// the recurrence's three, and no state update unless the final state is
// asked for.  Where S <= 16 and 2N = 4P (the bench's N = 128, P = 64) one
// launch of mamba_scan_kernel does everything, each head also convolving its
// group's B/C channels and forming G itself (the FUSED form below); else two
// kernels:
//   mamba_group_kernel, one workgroup per (sequence, group): the conv + SiLU
//     outputs of the group's B and C channels, [S][2N] fp32, and
//     G[s][j] = C_s . B_j, into the workspace -- shared by the group's heads;
//   mamba_scan_kernel, one workgroup of P/16 waves per (sequence, head): the
//     fp32 seed H0 (most of the HBM traffic) is loaded straight into the
//     registers of the fp32 matrix-core operand layout, the head's x
//     channels go through the conv into LDS, the group's B/C outputs are
//     copied in (C scaled by the decay exp(cum_s)), and
//     M[s][j] = dt_j exp(cum_s - cum_j) G[s][j]; each wave then forms a
//     16-row x 16-slot output tile as H0 C'^T + X^T M^T with
//     v_mfma_f32_16x16x4f32 and adds D x_s.  Optionally (the context tower
//     taking a committed block) the final state exp(cum_S) H0 +
//     sum_j dt_j exp(cum_S - cum_j) x_j B_j^T is written back (in place
//     allowed: every thread has read its part) and the conv state becomes
//     the block's last W-1 inputs (to a separate buffer: the B/C channels are
//     read by every head of the group).
#include <math.h>

#include <type_traits>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kMThreads = 256;
// a native 4-float vector: arrays of it stay in registers (arrays of HIP's
// float4 struct were left in scratch memory)
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ld_elt(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float ld_elt(const float* p, int64_t i) { return p[i]; }
// raw bits of one element (converted later by raw_f32), so that nothing
// between a load and its use needs the loaded register
__device__ __forceinline__ uint32_t ld_raw(const uint16_t* p) { return *p; }
__device__ __forceinline__ uint32_t ld_raw(const float* p) { return __float_as_uint(*p); }
template <typename T>
__device__ __forceinline__ float raw_f32(uint32_t r) {
  return std::is_same<T, float>::value ? __uint_as_float(r) : __uint_as_float(r << 16);
}
__device__ __forceinline__ void st_elt(uint16_t* p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}
__device__ __forceinline__ void st_elt(float* p, int64_t i, float v) { p[i] = v; }

// SiLU with the hardware reciprocal (about 1 ulp) instead of an IEEE
// divide; v -> -inf gives v * rcp(inf) = -0
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }
__device__ __forceinline__ float softplus(float v) { return v > 20.f ? v : log1pf(expf(v)); }

// Slots are handled in rounds of 16 (one 16 x 16 output tile per wave).
constexpr int kSC = 16;

// The pre-convolution inputs of `nch` channels for the window rows
// rw in [rw0, rw1) (rw = t + KW-1; t < 0 is the conv state, t >= 0 the
// block), as fp32 into LDS at dst[rw * stride + cc]; channel cc is global
// channel chan(cc).  Every load is unconditional (indexes past the end are
// clamped onto the last element and their values dropped), so the kU loads
// of a thread are in flight together and the thread waits once.
template <typename T, int KW, int NT, int nch, int kU, typename ChanFn>
__device__ __forceinline__ void load_window(const T* xbc, const T* cst, int C, int rw0, int rw1,
                                            ChanFn chan, float* dst, int stride) {
  const int total = (rw1 - rw0) * nch;
  for (int base = 0; base < total; base += kU * NT) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(base + u * NT + static_cast<int>(threadIdx.x), total - 1);
      const int r = rw0 + i / nch, cc = i % nch, c = chan(cc);
      const int t = r - (KW - 1);
      const T* src = t < 0 ? cst + static_cast<int64_t>(c) * (KW - 1) + r
                           : xbc + static_cast<int64_t>(t) * C + c;
      v[u] = ld_raw(src);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load before the first store
#pragma unroll
    for (int u = 0; u < kU; ++u) {     // clamped like the loads (same bytes as the owner)
      const int i = min(base + u * NT + static_cast<int>(threadIdx.x), total - 1);
      dst[(rw0 + i / nch) * stride + i % nch] = raw_f32<T>(v[u]);
    }
  }
}

// Conv + SiLU of `nch` channels over the S slots from a loaded window:
// out[s * ostride + cc] = SiLU(b[c] + sum_j w[c][j] win[(s + j) * stride + cc]).
// nch divides the thread count NT, so each thread keeps one channel and its
// taps.
// The conv taps and bias of the thread's channel (channel threadIdx.x % nch).
template <int KW>
struct Taps {
  float w[KW];
  float bias;
  __device__ __forceinline__ void load(const float* conv_w, const float* conv_b, int c) {
#pragma unroll
    for (int j = 0; j < KW; ++j) w[j] = conv_w[static_cast<int64_t>(c) * KW + j];
    bias = conv_b ? conv_b[c] : 0.f;
  }
};

// Conv + SiLU of `nch` channels over the S slots from a loaded window:
// out[s * ostride + cc] = SiLU(b[c] + sum_j w[c][j] win[(s + j) * stride + cc]).
// nch divides the thread count NT, so each thread keeps one channel and its
// taps (cc = threadIdx.x % nch).
template <int KW, int NT, int nch>
__device__ __forceinline__ void conv_window(const float* win, int stride, int S, const Taps<KW>& tp,
                                            float* out, int ostride) {
  static_assert(NT % nch == 0, "one channel per thread");
  const int cc = threadIdx.x % nch;
  for (int si = threadIdx.x / nch; si < S; si += NT / nch) {
    float acc = tp.bias;
#pragma unroll
    for (int j = 0; j < KW; ++j) acc = fmaf(tp.w[j], win[(si + j) * stride + cc], acc);
    out[si * ostride + cc] = silu(acc);
  }
}

// Per (sequence, group): the conv outputs of the group's B and C channels,
// [S][2N] fp32, and G[s][j] = C_s . B_j for j <= s, 0 elsewhere, as
// [Sp][Sp] (S rounded up to 16) -- the parts every head of the group
// shares.
template <typename T, int N, int KW>
__global__ __launch_bounds__(kMThreads) void mamba_group_kernel(MambaArgs a, float* ws_bc, float* ws_g) {
  const int b = blockIdx.x / a.G;
  const int g = blockIdx.x % a.G;
  if (a.active && !a.active[b]) return;
  const int S = a.S, H = a.H, G = a.G, P = a.P;
  const int Sp = (S + kSC - 1) / kSC * kSC;
  const int C = H * P + 2 * G * N;
  constexpr int BCP = 2 * N + 4;         // LDS row stride (rows start 4 banks apart)
  // one batch of loads covers the window of 16 slots
  constexpr int kU = ((kSC + KW - 1) * 2 * N + kMThreads - 1) / kMThreads;
  extern __shared__ float lds[];
  float* win = lds;                      // [S + KW-1][BCP]
  float* out = lds + (S + KW - 1) * BCP; // [S][BCP]
  const T* xbc = static_cast<const T*>(a.xbc) + static_cast<int64_t>(b) * S * C;
  const T* cst = static_cast<const T*>(a.conv_state) + static_cast<int64_t>(b) * C * (KW - 1);
  auto chan = [&](int cc) { return H * P + (cc < N ? g * N + cc : G * N + g * N + (cc - N)); };
  Taps<KW> tp;
  tp.load(a.conv_w, a.conv_b, chan(threadIdx.x % (2 * N)));
  // One thread per B/C channel and S <= 16: element u * 2N + tid of the
  // window is row u of channel tid, so the thread's own loads hold its
  // channel's whole window and the conv runs from registers (rows past
  // the window load a clamped element and are never used).
  if (kMThreads == 2 * N && S <= kSC) {
    constexpr int kRows = kSC + KW - 1;
    const int tid = threadIdx.x;
    const int total = (S + KW - 1) * 2 * N;
    uint32_t v[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int i = min(u * 2 * N + tid, total - 1);
      const int r = i / (2 * N), c = chan(i % (2 * N));
      const int t = r - (KW - 1);
      const T* src = t < 0 ? cst + static_cast<int64_t>(c) * (KW - 1) + r
                           : xbc + static_cast<int64_t>(t) * C + c;
      v[u] = ld_raw(src);
    }
#pragma unroll
    for (int si = 0; si < kSC; ++si) {   // unrolled: constant register indexes
      if (si < S) {
        float acc = tp.bias;
#pragma unroll
        for (int j = 0; j < KW; ++j) acc = fmaf(tp.w[j], raw_f32<T>(v[si + j]), acc);
        out[si * BCP + tid] = silu(acc);
      }
    }
  } else {
    load_window<T, KW, kMThreads, 2 * N, kU>(xbc, cst, C, 0, S + KW - 1, chan, win, BCP);
    __syncthreads();
    conv_window<KW, kMThreads, 2 * N>(win, BCP, S, tp, out, BCP);
  }
  __syncthreads();
  float* bc = ws_bc + (static_cast<int64_t>(b) * G + g) * S * 2 * N;
  for (int i = threadIdx.x; i < S * 2 * N / 4; i += kMThreads) {
    const int si = (4 * i) / (2 * N), cc = (4 * i) % (2 * N);
    *reinterpret_cast<float4*>(bc + 4 * i) = *reinterpret_cast<const float4*>(out + si * BCP + cc);
  }
  float* gm = ws_g + (static_cast<int64_t>(b) * G + g) * Sp * Sp;
  // (si, j) pairs, 16 j per pass over a row (no division by the runtime S)
  for (int si = threadIdx.x >> 4; si < Sp; si += kMThreads >> 4)
    for (int j = threadIdx.x & 15; j < Sp; j += 16) {
      float d = 0.f;
      if (j <= si && si < S) {
        const float* cs = out + si * BCP + N;
        const float* bs = out + j * BCP;
#pragma unroll 4
        for (int n = 0; n < N; n += 4) {
          const float4 x4 = *reinterpret_cast<const float4*>(cs + n);
          const float4 y4 = *reinterpret_cast<const float4*>(bs + n);
          d = fmaf(x4.x, y4.x, fmaf(x4.y, y4.y, fmaf(x4.z, y4.z, fmaf(x4.w, y4.w, d))));
        }
      }
      gm[si * Sp + j] = d;
    }
}

// The global inputs of one round of 16 slots of the scan kernel: the
// group's B/C rows, the head's x window rows and the G rows, held in
// registers (the caller's arrays) between their loads and their LDS stores.
template <typename T, int P, int N, int KW, int NT>
struct ScanRound {
  static constexpr int kBC = (kSC * 2 * N / 4 + NT - 1) / NT;       // float4 of B/C rows
  static constexpr int kWn = ((kSC + KW - 1) * P + NT - 1) / NT;    // window elements
  static constexpr int kG = (kSC * 64 / 4 + NT - 1) / NT;           // float4 of G rows (Sp <= 64)

  // window rows [rw0, rw1) of round r0: round 0 also takes the W-1 rows of
  // the conv state
  static __device__ __forceinline__ int rw0(int r0) { return r0 == 0 ? 0 : r0 + KW - 1; }
  static __device__ __forceinline__ int rw1(int r0, int S) { return min(r0 + kSC, S) + KW - 1; }

  // the head's x window rows of the round
  static __device__ __forceinline__ void issue_x(uint32_t (&w)[kWn], const T* xbc, const T* cst, int C,
                                                 int h, int S, int r0) {
    const int tid = threadIdx.x;
    const int w0 = rw0(r0), nw = (rw1(r0, S) - w0) * P;
#pragma unroll
    for (int u = 0; u < kWn; ++u) {
      const int i = min(u * NT + tid, nw - 1);
      const int r = w0 + i / P, c = h * P + i % P;
      const int t = r - (KW - 1);
      const T* src = t < 0 ? cst + static_cast<int64_t>(c) * (KW - 1) + r
                           : xbc + static_cast<int64_t>(t) * C + c;
      w[u] = ld_raw(src);
    }
  }

  static __device__ __forceinline__ void issue(v4f (&bc)[kBC], uint32_t (&w)[kWn], v4f (&gv)[kG],
                                               const float* bcg, const float* gmg, const T* xbc,
                                               const T* cst, int C, int h, int S, int Sp, int r0) {
    const int tid = threadIdx.x;
    const int nbc = (min(r0 + kSC, S) - r0) * 2 * N / 4;
#pragma unroll
    for (int u = 0; u < kBC; ++u)
      bc[u] = reinterpret_cast<const v4f*>(bcg + r0 * 2 * N)[min(u * NT + tid, nbc - 1)];
    issue_x(w, xbc, cst, C, h, S, r0);
    const int ng = kSC * Sp / 4;           // 16 rows of G, each Sp wide
#pragma unroll
    for (int u = 0; u < kG; ++u)
      gv[u] = reinterpret_cast<const v4f*>(gmg + r0 * Sp)[min(u * NT + tid, ng - 1)];
  }

  // Unconditional stores with the loads' clamped indexes: a lane past the
  // end writes the last element's value to the last element's place (the
  // same bytes its owner writes).  A conditional store would let the
  // compiler sink each load into its branch, one wait per load.
  static __device__ __forceinline__ void commit_x(const uint32_t (&w)[kWn], float* s_win, int S, int r0,
                                                  int XP) {
    const int tid = threadIdx.x;
    const int w0 = rw0(r0), nw = (rw1(r0, S) - w0) * P;
#pragma unroll
    for (int u = 0; u < kWn; ++u) {
      const int i = min(u * NT + tid, nw - 1);
      s_win[(w0 + i / P) * XP + i % P] = raw_f32<T>(w[u]);
    }
  }

  static __device__ __forceinline__ void commit(const v4f (&bc)[kBC], const uint32_t (&w)[kWn],
                                                const v4f (&gv)[kG], float* s_b, int c_off,
                                                float* s_win, float* s_m, int S, int Sp, int r0,
                                                int BP, int XP) {
    const int tid = threadIdx.x;
    const int nbc = (min(r0 + kSC, S) - r0) * 2 * N / 4;
#pragma unroll
    for (int u = 0; u < kBC; ++u) {
      const int i = min(u * NT + tid, nbc - 1);
      const int si = r0 + (4 * i) / (2 * N), cc = (4 * i) % (2 * N);
      // B channels to s_b, C channels to s_b + c_off (a select, not a branch)
      const int off = si * BP + cc + (cc >= N ? c_off - N : 0);
      *reinterpret_cast<v4f*>(s_b + off) = bc[u];
    }
    commit_x(w, s_win, S, r0, XP);
    const int ng = kSC * Sp / 4;
#pragma unroll
    for (int u = 0; u < kG; ++u)
      reinterpret_cast<v4f*>(s_m + r0 * Sp)[min(u * NT + tid, ng - 1)] = gv[u];
  }
};

// Per (sequence, head): P/16 waves; wave w owns state rows 16w..16w+15, lane
// l row p = 16w + l%16 and KS = N/4 entries of it: n = 16 (t/4) + 4 kg + t%4
// for its t-th entry, kg = l/16.  The outputs of 16 slots at a time are one 16 x 16 fp32 matrix
// tile per wave, accumulated by v_mfma_f32_16x16x4f32 in two parts:
//   H0 C_s               -- K = N, taken in the order of the lanes' own
//                            entries: at step t each lane's A operand is its
//                            state entry t and its B operand C[s][n] for the
//                            same n; the tile is then scaled by the decay
//                            exp(cum_s);
//   X^T M^T              -- K = the slots j (4 per step), the in-block sum
//                            sum_j M[s][j] x_j[p] (M is 0 for j > s).
// Lane l then holds y at slot s0 + l%16 for rows 16w + 4 kg + r, r < 4.
// Global loads: the round's inputs first, then the seed's state (most of
// the bytes) -- waiting for the former leaves the latter in flight.
// CTX: the context tower's form (final SSM state written; its own
// instantiation, so that the denoiser's form keeps its smaller register
// allocation)
// FUSED (S <= 16 and one thread per B/C channel, NT == 2N): the kernel
// also does the group kernel's part for its own head -- the conv + SiLU of
// the group's B/C channels from registers, and G = C B^T on the matrix cores,
// each wave over N/(P/16) state entries, its partial tile summed in LDS --
// so one launch does the whole layer and the workspace is not used.  The
// B/C window is read by all H/G heads of the group, which the XCD-aware
// order below runs on one XCD, so seven of the eight reads hit its L2.
template <typename T, int P, int N, int KW, bool CTX, bool FUSED>
__global__ __launch_bounds__(4 * P) void mamba_scan_kernel(MambaArgs a, const float* ws_bc,
                                                          const float* ws_g) {
  constexpr int NT = 4 * P;              // P/16 waves of 64
  constexpr int KS = N / 4;              // state entries per lane
  static_assert(KS % 4 == 0, "16-byte state loads");
  static_assert(!FUSED || NT == 2 * N, "one thread per B/C channel");
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  // XCD-aware order: workgroups go to the 8 XCDs round-robin, so workgroup
  // i runs (sequence, head) unit (i % 8) * ceil(n/8) + i / 8 and the heads of
  // one group (consecutive units) share an XCD and its L2
  const int n_units = a.B * a.H;
  const int unit = (blockIdx.x % 8) * ((n_units + 7) / 8) + blockIdx.x / 8;
  if (unit >= n_units) return;
  const int b = unit / a.H;
  const int h = unit % a.H;
  if (a.active && !a.active[b]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S, H = a.H, G = a.G;
  const int Sp = (S + kSC - 1) / kSC * kSC; // slots rounded up to whole tiles (zero padded)
  constexpr int W = KW;
  const int g = h / (H / G);
  const int C = H * P + 2 * G * N;
  constexpr int XP = P + 4;              // LDS row strides (rows start 4 banks apart)
  constexpr int BP = N + 4;
  // FUSED with P = 64: the x conv runs from registers (no x window in LDS)
  constexpr bool kXinRegs = FUSED && P == 64;
  extern __shared__ float lds[];
  float* s_win = lds;                    // [S + W-1][XP]  x inputs
  float* s_x = s_win + (kXinRegs ? 0 : (S + W - 1) * XP); // [Sp][XP] conv outputs of the head's x
  float* s_b = s_x + Sp * XP;            // [Sp][BP]       the group's B
  float* s_c = s_b + Sp * BP;            // [Sp][BP]       the group's C
  float* s_dt = s_c + Sp * BP;           // [Sp] dt_s
  float* s_cum = s_dt + Sp;              // [Sp] sum_{k<=s} dt_k A  (log of the decay)
  float* s_dec = s_cum + Sp;             // [Sp] exp(cum_s), 0 past S
  float* s_m = s_dec + Sp;               // [Sp][Sp]  G, then dt_j exp(cum_s - cum_j) G[s][j]
  float* s_gp = s_m + Sp * Sp;           // FUSED: [P/16][16][16] the waves' partial G tiles
  const T* xbc = static_cast<const T*>(a.xbc) + static_cast<int64_t>(b) * S * C;
  const T* cst = static_cast<const T*>(a.conv_state) + static_cast<int64_t>(b) * C * (W - 1);
  const float* bcg = ws_bc + (static_cast<int64_t>(b) * G + g) * S * 2 * N;
  const float* gmg = ws_g + (static_cast<int64_t>(b) * G + g) * Sp * Sp;

  // ---- global loads: dt of slot `lane`, round 0's inputs, the seed state
  const float dtr = a.dt_raw[(static_cast<int64_t>(b) * S + min(lane, S - 1)) * H + h];
  const float A = -expf(a.A_log[h]);
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.f;
  const float Dh = a.D ? a.D[h] : 0.f;
  Taps<KW> tp;
  tp.load(a.conv_w, a.conv_b, h * P + tid % P);
  using RD = ScanRound<T, P, N, KW, NT>;
  const int pl = lane & 15, kg = lane >> 4;
  const int p = wave * 16 + pl;
  // the lane's state entries, row p: n = 16 (t/4) + 4 kg + t%4 (the output
  // layout of the final state's matrix products below; any order of K
  // serves H0 C^T as long as C is read in the same one).  Each 16-byte load
  // of a wave then covers 64 consecutive bytes of each of its 16 rows: 16
  // cache lines per load instruction, half of each, where runs of KS
  // entries per lane touched 64 lines a sixteenth at a time (measured 2 us
  // faster from HBM at the bench shape).
  constexpr int kStride = 4;             // distance in n between consecutive float4 of a lane
  const int64_t sbase = ((static_cast<int64_t>(b) * H + h) * P + p) * N + 4 * kg;
  float st[KS];
  auto load_state = [&]() {
#pragma unroll
    for (int j = 0; j < KS; j += 4) {
      const float4 v = *reinterpret_cast<const float4*>(a.ssm_state + sbase + kStride * j);
      st[j] = v.x; st[j + 1] = v.y; st[j + 2] = v.z; st[j + 3] = v.w;
    }
  };
  if constexpr (FUSED) {
    // the thread's B/C channel cb over the window rows (clamped onto the
    // last row; rows past the window only feed slots past S), its taps, and
    // the head's x window
    constexpr int kRows = kSC + KW - 1;
    const int cb = H * P + (tid < N ? g * N + tid : G * N + g * N + (tid - N));
    Taps<KW> tb;
    tb.load(a.conv_w, a.conv_b, cb);
    // x, P = 64: wave w convolves slots 4w .. 4w+3 of channel c = lane from
    // its own registers (window rows 4w .. 4w+2+W, clamped onto the last),
    // so the x window needs no LDS; the row pointers are uniform and a load
    // needs no address arithmetic of its own; rows below W-1 (wave 0 only)
    // come from the conv state
    constexpr int kXR = 4 + KW - 1;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t xw[kXinRegs ? kXR : 1];
    uint32_t w[kXinRegs ? 1 : RD::kWn];
    if constexpr (kXinRegs) {
      const int c = h * P + lane;
#pragma unroll
      for (int u = 0; u < kXR; ++u) {
        const int r = min(4 * wv + u, S + KW - 2);
        const T* src;
        if (u < KW - 1)
          src = r < KW - 1 ? cst + static_cast<int64_t>(c) * (KW - 1) + r
                           : xbc + static_cast<int64_t>(r - (KW - 1)) * C + c;
        else
          src = xbc + static_cast<int64_t>(r - (KW - 1)) * C + c;
        xw[u] = ld_raw(src);
      }
    } else {
      RD::issue_x(w, xbc, cst, C, h, S, 0);
    }
    // B/C window: rows u < W-1 from the conv state, the others slot
    // min(u - (W-1), S-1) of the block (uniform row pointers)
    uint32_t vb[kRows];
    const T* cs_ch = cst + static_cast<int64_t>(cb) * (KW - 1);
#pragma unroll
    for (int u = 0; u < KW - 1; ++u) vb[u] = ld_raw(cs_ch + u);
#pragma unroll
    for (int u = KW - 1; u < kRows; ++u) {
      const T* row = xbc + static_cast<int64_t>(min(u - (KW - 1), S - 1)) * C;
      vb[u] = ld_raw(row + cb);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_state();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kXinRegs) {
      // slots past S are stored as 0 (the zero padding of s_x)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float acc = tp.bias;
#pragma unroll
        for (int j = 0; j < KW; ++j) acc = fmaf(tp.w[j], raw_f32<T>(xw[q + j]), acc);
        s_x[(4 * wv + q) * XP + lane] = 4 * wv + q < S ? silu(acc) : 0.f;
      }
    } else {
      RD::commit_x(w, s_win, S, 0, XP);
    }
    // conv + SiLU of the channel; slots past S are stored as 0
    float* dst = tid < N ? s_b + tid : s_c + (tid - N);
#pragma unroll
    for (int si = 0; si < kSC; ++si) {
      float acc = tb.bias;
#pragma unroll
      for (int j = 0; j < KW; ++j) acc = fmaf(tb.w[j], raw_f32<T>(vb[si + j]), acc);
      dst[si * BP] = si < S ? silu(acc) : 0.f;
    }
  } else {
    {
      v4f bc[RD::kBC];
      uint32_t w[RD::kWn];
      v4f gv[RD::kG];
      RD::issue(bc, w, gv, bcg, gmg, xbc, cst, C, h, S, Sp, 0);
      // a scheduling fence keeps the round's loads ahead of the state's, so
      // that waiting for the former leaves the latter in flight
      __builtin_amdgcn_sched_barrier(0);
      load_state();
      __builtin_amdgcn_sched_barrier(0);
      RD::commit(bc, w, gv, s_b, Sp * BP, s_win, s_m, S, Sp, 0, BP, XP);
    }
    for (int r0 = kSC; r0 < S; r0 += kSC) {
      v4f bc[RD::kBC];
      uint32_t w[RD::kWn];
      v4f gv[RD::kG];
      RD::issue(bc, w, gv, bcg, gmg, xbc, cst, C, h, S, Sp, r0);
      RD::commit(bc, w, gv, s_b, Sp * BP, s_win, s_m, S, Sp, r0, BP, XP);
    }
  }
  // dt, and the decay's log as an inclusive prefix sum over the slots
  // (wave 0, lane = slot; S <= 64)
  if (wave == 0) {
    const float dt = softplus(dtr + dtb);
    float cum = lane < S ? dt * A : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float v = __shfl_up(cum, o);
      if (lane >= o) cum += v;
    }
    if (lane < Sp) {
      s_dt[lane] = dt;
      s_cum[lane] = cum;
      s_dec[lane] = lane < S ? expf(cum) : 0.f;
    }
  }
  __syncthreads();
  if constexpr (!kXinRegs) {
    conv_window<KW, NT, P>(s_win, XP, S, tp, s_x, XP);
    for (int i = tid; i < (Sp - S) * XP; i += NT) s_x[S * XP + i] = 0.f;
  }
  if constexpr (FUSED) {
    // this wave's part of G = C B^T (16 x 16, Sp = 16): D[s][j] over the
    // entries n in [wave KW4, wave KW4 + KW4), lane group kg taking KQ
    // consecutive ones; A = C[s = lane%16][n], B = B_j[n] for j = lane%16
    constexpr int KW4 = N / (P / 16), KQ = KW4 / 4;
    static_assert(KQ % 4 == 0, "16-byte operand reads");
    const float* ca = s_c + pl * BP + wave * KW4 + kg * KQ;
    const float* ba = s_b + pl * BP + wave * KW4 + kg * KQ;
    f32x4 gd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KQ; t += 4) {
      const float4 cv = *reinterpret_cast<const float4*>(ca + t);
      const float4 bv = *reinterpret_cast<const float4*>(ba + t);
      gd = __builtin_amdgcn_mfma_f32_16x16x4f32(cv.x, bv.x, gd, 0, 0, 0);
      gd = __builtin_amdgcn_mfma_f32_16x16x4f32(cv.y, bv.y, gd, 0, 0, 0);
      gd = __builtin_amdgcn_mfma_f32_16x16x4f32(cv.z, bv.z, gd, 0, 0, 0);
      gd = __builtin_amdgcn_mfma_f32_16x16x4f32(cv.w, bv.w, gd, 0, 0, 0);
    }
    // lane: column j = lane%16, rows s = 4 kg + r
#pragma unroll
    for (int r = 0; r < 4; ++r) s_gp[wave * 256 + (4 * kg + r) * 16 + pl] = gd[r];
    __syncthreads();
  }
  for (int si = tid >> 4; si < Sp; si += NT >> 4)
    for (int j = tid & 15; j < Sp; j += 16) {
      float* m = s_m + si * Sp + j;
      float gsj;
      if constexpr (FUSED) {             // the waves' partials, in wave order
        gsj = s_gp[si * 16 + j];
#pragma unroll
        for (int q = 1; q < P / 16; ++q) gsj += s_gp[q * 256 + si * 16 + j];
      } else {
        gsj = *m;
      }
      *m = (j <= si && si < S) ? s_dt[j] * __expf(s_cum[si] - s_cum[j]) * gsj : 0.f;
    }
  __syncthreads();

  // ---- outputs, one 16-slot tile at a time
  T* y = static_cast<T*>(a.y) + (static_cast<int64_t>(b) * S) * (H * P) + h * P + wave * 16 + 4 * kg;
  for (int s0 = 0; s0 < Sp; s0 += kSC) {
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    const float* crow = s_c + (s0 + pl) * BP + 4 * kg;
#pragma unroll
    for (int t = 0; t < KS; t += 4) {
      const float4 cv = *reinterpret_cast<const float4*>(crow + kStride * t);
      d = __builtin_amdgcn_mfma_f32_16x16x4f32(st[t], cv.x, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x4f32(st[t + 1], cv.y, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x4f32(st[t + 2], cv.z, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x4f32(st[t + 3], cv.w, d, 0, 0, 0);
    }
    // rows of C past S hold stale values: they reach only the tile columns
    // of slots past S, which nothing stores
    const float dec = s_dec[s0 + pl];
    d *= dec;
    const float* mrow = s_m + (s0 + pl) * Sp;
    for (int j0 = 0; j0 < s0 + kSC; j0 += 4)
      d = __builtin_amdgcn_mfma_f32_16x16x4f32(s_x[(j0 + kg) * XP + p], mrow[j0 + kg], d, 0, 0, 0);
    const int si = s0 + pl;
    if (si < S) {
      const float4 xr = *reinterpret_cast<const float4*>(s_x + si * XP + wave * 16 + 4 * kg);
      const float o0 = d[0] + Dh * xr.x, o1 = d[1] + Dh * xr.y;
      const float o2 = d[2] + Dh * xr.z, o3 = d[3] + Dh * xr.w;
      T* yo = y + static_cast<int64_t>(si) * (H * P);
      if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<float4*>(yo) = make_float4(o0, o1, o2, o3);
      } else {
        const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o0)) |
                            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(o1))) << 16);
        const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o2)) |
                            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(o3))) << 16);
        *reinterpret_cast<uint2*>(yo) = make_uint2(lo, hi);
      }
    }
  }

  // ---- the context tower's final state: H_S = exp(cum_S) H0 +
  // sum_j dt_j exp(cum_S - cum_j) x_j B_j^T (in place allowed: every thread
  // has read its part), and the conv state = the last W-1 inputs
  // on the matrix cores: per 16-entry tile nt of n, the wave's 16 x 16
  // block of H_S^T = d0 H0^T + sum_j (w_j B_j)[16 nt + i] x_j[p], K = the
  // slots j four at a time, w_j = dt_j exp(cum_S - cum_j); the accumulator
  // starts from the lane's own state entries (d0 = exp(cum_S))
  if constexpr (CTX) {
    const float last = s_cum[S - 1];
    const float d0 = s_dec[S - 1];
    f32x4 hs[KS / 4];
#pragma unroll
    for (int nt = 0; nt < KS / 4; ++nt)
      hs[nt] = f32x4{st[4 * nt] * d0, st[4 * nt + 1] * d0, st[4 * nt + 2] * d0, st[4 * nt + 3] * d0};
    for (int j0 = 0; j0 < Sp; j0 += 4) {
      const int j = j0 + kg;
      // slots past S: a select, not a product (the LDS rows read there may
      // be stale); x is 0 there
      const float w = j < S ? s_dt[j] * expf(last - s_cum[j]) : 0.f;
      const float xv = s_x[j * XP + p];
      const float* brow = s_b + j * BP + pl;
#pragma unroll
      for (int nt = 0; nt < KS / 4; ++nt) {
        const float av = j < S ? brow[16 * nt] * w : 0.f;
        hs[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, xv, hs[nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int nt = 0; nt < KS / 4; ++nt)
      *reinterpret_cast<float4*>(a.ssm_state_out + sbase + 16 * nt) =
          make_float4(hs[nt][0], hs[nt][1], hs[nt][2], hs[nt][3]);
  }
  if (a.conv_state_out) {
    T* cso = static_cast<T*>(a.conv_state_out) + static_cast<int64_t>(b) * C * (W - 1);
    // x channels by their head; B and C channels by the group's first head
    const bool owns_bc = (h % (H / G)) == 0;
    constexpr int CH = P + 2 * N;
    for (int cl = tid; cl < CH; cl += NT) {
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
hipError_t launch_t(const MambaArgs& a, void* ws, hipStream_t st) {
  const size_t lds_g = mamba_group_lds_bytes(a.S, a.N);
  const size_t lds_s = mamba_lds_bytes(a.S, a.P, a.N);
  float* ws_bc = static_cast<float*>(ws);
  float* ws_g = ws_bc + static_cast<size_t>(a.B) * a.G * a.S * 2 * a.N;
  const dim3 blk(kMThreads);
  // more than 64 KB of dynamic LDS must be allowed per kernel (up to 160 KB)
  auto allow = [](const void* f, size_t bytes) {
    return bytes > 65536 ? hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(bytes))
                         : hipSuccess;
  };
  // the XCD-aware grid: 8 * ceil(units / 8) workgroups
  const dim3 grid(static_cast<unsigned>((a.B * a.H + 7) / 8 * 8));
  // one launch (FUSED) where it applies, else the group kernel and the scan
#define TT_SCAN(PP, NN, WW, CTX, FUSED)                                                         \
  {                                                                                             \
    hipError_t e = allow(reinterpret_cast<const void*>(&mamba_scan_kernel<T, PP, NN, WW, CTX, FUSED>), lds_s); \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL((mamba_scan_kernel<T, PP, NN, WW, CTX, FUSED>), grid, dim3(4 * PP), lds_s, \
                       st, a, ws_bc, ws_g);                                                     \
    return hipGetLastError();                                                                   \
  }
#define TT_MAMBA(PP, NN, WW)                                                                    \
  if (a.P == PP && a.N == NN && a.W == WW) {                                                    \
    if constexpr (4 * PP == 2 * NN) {                                                           \
      if (mamba_fused(a.S, PP, NN)) {                                                           \
        if (a.ssm_state_out) TT_SCAN(PP, NN, WW, true, true)                                    \
        TT_SCAN(PP, NN, WW, false, true)                                                        \
      }                                                                                         \
    }                                                                                           \
    hipError_t e = allow(reinterpret_cast<const void*>(&mamba_group_kernel<T, NN, WW>), lds_g); \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL((mamba_group_kernel<T, NN, WW>), dim3(static_cast<unsigned>(a.B * a.G)), \
                       blk, lds_g, st, a, ws_bc, ws_g);                                         \
    e = hipGetLastError();                                                                      \
    if (e != hipSuccess) return e;                                                              \
    if (a.ssm_state_out) TT_SCAN(PP, NN, WW, true, false)                                       \
    TT_SCAN(PP, NN, WW, false, false)                                                           \
  }
#define TT_MAMBA_W(PP, NN) TT_MAMBA(PP, NN, 2) TT_MAMBA(PP, NN, 3) TT_MAMBA(PP, NN, 4)
  TT_MAMBA_W(64, 128)
  TT_MAMBA_W(64, 64)
  TT_MAMBA_W(32, 128)
  TT_MAMBA_W(32, 64)
#undef TT_MAMBA_W
#undef TT_MAMBA
#undef TT_SCAN
  return hipErrorInvalidValue;
}

}  // namespace

bool mamba_fused(int S, int P, int N) { return S <= kSC && 4 * P == 2 * N; }

bool mamba_supported(int P, int N, int W) {
  return (P == 64 || P == 32) && (N == 128 || N == 64) && W >= 2 && W <= 4;
}

size_t mamba_lds_bytes(int S, int P, int N) {
  // the scan kernel: the x window (S + 3 rows at most) and outputs (S
  // rounded up to 16), B and C rows (S rounded up), dt, cum, M and, in the
  // one-launch form, the waves' partial G tiles; the group kernel needs
  // (2S + 3) (2N + 4) floats, checked separately
  const size_t Sp = (S + 15) / 16 * 16;
  const bool fused = mamba_fused(S, P, N);
  const size_t gp = fused ? static_cast<size_t>(P / 16) * 256 : 0;
  const size_t win = fused && P == 64 ? 0 : static_cast<size_t>(S + 3);   // x window rows
  return (static_cast<size_t>(win + Sp) * (P + 4) + 2 * Sp * (N + 4) + 3 * Sp + Sp * Sp + gp) *
         sizeof(float);
}

size_t mamba_group_lds_bytes(int S, int N) {
  return static_cast<size_t>(2 * S + 3) * (2 * N + 4) * sizeof(float);
}

size_t mamba_workspace_bytes(int B, int S, int G, int N) {
  // per (sequence, group): the B/C conv outputs [S][2N] and G [Sp][Sp]
  const size_t Sp = (S + 15) / 16 * 16;
  return static_cast<size_t>(B) * G * (static_cast<size_t>(S) * 2 * N + Sp * Sp) * sizeof(float);
}

hipError_t launch_mamba_scan(const MambaArgs& a, void* ws, hipStream_t st) {
  return a.dtype == 0 ? launch_t<uint16_t>(a, ws, st) : launch_t<float>(a, ws, st);
}

}  // namespace tt
