// The denoiser's weighted adaLN-single attention sublayer around the block
// attention:
//   h   = LayerNorm(x) (1 + scale_b) + shift_b       ln_modulate_kernel
//   q|k|v = h W_qkv^T                                gemm_kernel<kEpiQkv>
//   o   = block attention (the attention kernels, identity modulation)
//   out = x + gate_b (o W_o^T)                       gemm_kernel<kEpiGate>
// [dothoosh] two-tower mechanism section and [modelcard] technical features:
// every denoiser layer takes a timestep scale, shift and gate through
// adaLN-single; the layer around them follows the published adaLN-single
// placement (PixArt-alpha / DiT): LayerNorm without affine (eps 1e-6), the
// modulation, bias-free projections, the gate on the projected attention
// output before the residual add.
//
// ln_modulate_kernel: one wave per token row; the row stays in registers
// (bf16, up to 8192 wide), mean and variance by exact two-pass sums and
// wave reductions, output bf16 (the projection's operand).
//
// gemm_kernel: C[M, N] = A[M, K] W[N, K]^T in bf16 with fp32 accumulation
// on the matrix cores (v_mfma_f32_32x32x16_bf16).  One workgroup of 4 waves
// per 128 x 128 output tile; K in steps of 64.  A and W tiles stream
// HBM -> LDS through the direct copy path into an NS-stage ring (NS - 1
// steps in flight while one is multiplied; NS = 3 when the tiles fit one
// per CU, else 2 so that two tiles share a CU).  LDS rows are 128 bytes (64 k); the
// 16-byte slot of k-chunk c in row r is c ^ ((r >> 1) & 7), so the 16 rows
// read together by a matrix-operand load hit 16 different bank groups.
// Each wave computes a 64 x 64 piece as the transpose C^T = W A^T: the A
// operand is 32 W rows x 16 k, the B operand 32 A rows x 16 k, so a lane's
// 16 accumulators are 4 runs of 4 consecutive output columns of one output
// row, stored as 8-byte groups by the epilogues.  Tiles are numbered
// M-fastest and handed out in contiguous ranges per XCD (workgroup i runs
// on XCD i % 8), so the tiles that share W columns share an L2.
#include <math.h>

#include <atomic>

#include "tt_internal.h"

namespace tt {
namespace {

#define TT_LDS __attribute__((address_space(3)))
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGThreads = 256;
constexpr int kTileBytes = kBM * kBK * 2;         // one operand tile: 16 KB
constexpr int kStageBytes = 2 * kTileBytes;       // A tile, then W tile
constexpr int kCopies = kTileBytes / 1024 / 4;    // 1 KB copies per wave per operand tile

enum { kEpiQkv = 0, kEpiGate = 1 };

// 16-byte global -> LDS copy through the direct path from a wave-uniform
// base plus a per-lane byte offset: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16).  In asm so that the compiler does not wait
// for the copies in flight before every LDS read; the stage waits are
// explicit.  No register result.  M0 is not in the clobber list (the
// compiler reserves it and warns that such a clobber is not honoured); the
// build fails if the compiler itself uses M0 in this file's kernels.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds) : "memory");
}

// Waits until at most N vector memory operations of this wave are in flight.
// The stage waits count the copies only: the loops that use them issue no
// other vector memory operation (operands come from LDS and registers; the
// build checks that the kernels neither spill nor use M0 elsewhere).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// wait until at most `later` pipeline steps' copies (2 kCopies each) of
// this wave are in flight (later <= NS - 2, wave-uniform; <= 0: all done)
template <int NS>
__device__ __forceinline__ void wait_steps(int later) {
  constexpr int c = 2 * kCopies;
  static_assert(NS >= 2 && NS <= 4, "ring of 2 to 4 stages");
  if (NS == 2 || later <= 0) wait_vmem<0>();
  else if (NS == 3 || later == 1) wait_vmem<c>();
  else wait_vmem<2 * c>();
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ------------------------------------------------------- LayerNorm + modulate
template <int NCH>
__global__ __launch_bounds__(256) void ln_modulate_kernel(LnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + wave;
  if (m >= a.M) return;
  const int b = m / a.S;
  if (a.active && !a.active[b]) return;
  const int D = a.D;
  const uint16_t* xr = a.x + static_cast<int64_t>(m) * D;
  // 8 channels per lane per 512-wide chunk; the tail chunk's lanes past D
  // load the row's last 8 channels (dropped below)
  uint4 raw[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    raw[c] = *reinterpret_cast<const uint4*>(xr + min(c * 512 + lane * 8, D - 8));
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c * 512 + lane * 8 < D) {
      const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) s += bf_lo(w[i]) + bf_hi(w[i]);
    }
  }
  const float mean = wave_sum(s) / static_cast<float>(D);
  float v = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c * 512 + lane * 8 < D) {
      const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d0 = bf_lo(w[i]) - mean, d1 = bf_hi(w[i]) - mean;
        v = fmaf(d0, d0, fmaf(d1, d1, v));
      }
    }
  }
  const float rstd = 1.f / sqrtf(wave_sum(v) / static_cast<float>(D) + 1e-6f);
  const float* sh = a.shift + static_cast<int64_t>(b) * D;
  const float* sc = a.scale + static_cast<int64_t>(b) * D;
  uint16_t* hr = a.h + static_cast<int64_t>(m) * D;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = c * 512 + lane * 8;
    if (col < D) {
      const float4 s0 = *reinterpret_cast<const float4*>(sh + col);
      const float4 s1 = *reinterpret_cast<const float4*>(sh + col + 4);
      const float4 k0 = *reinterpret_cast<const float4*>(sc + col);
      const float4 k1 = *reinterpret_cast<const float4*>(sc + col + 4);
      const float shv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      const float scv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y0 = fmaf((bf_lo(w[i]) - mean) * rstd, 1.f + scv[2 * i], shv[2 * i]);
        const float y1 = fmaf((bf_hi(w[i]) - mean) * rstd, 1.f + scv[2 * i + 1], shv[2 * i + 1]);
        o[i] = pack2(y0, y1);
      }
      *reinterpret_cast<uint4*>(hr + col) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// The epilogues for the 4 output columns n..n+3 of row m (sequence b):
// kEpiQkv scatters them to q, k or v (a group never straddles: the
// boundaries are multiples of 64); kEpiGate writes x + gate * C.
template <int EPI>
__device__ __forceinline__ void store4(const GemmArgs& a, int m, int b, int n, float c0, float c1,
                                       float c2, float c3) {
  if constexpr (EPI == kEpiQkv) {
    uint16_t* dst;
    if (n < a.nq) dst = a.q + static_cast<int64_t>(m) * a.nq + n;
    else if (n < a.nq + a.nk) dst = a.k + static_cast<int64_t>(m) * a.nk + (n - a.nq);
    else dst = a.v + static_cast<int64_t>(m) * a.nk + (n - a.nq - a.nk);
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(c0, c1), pack2(c2, c3));
  } else {
    const int64_t o = static_cast<int64_t>(m) * a.N + n;
    const uint2 xv = *reinterpret_cast<const uint2*>(a.x + o);
    const float4 gv = *reinterpret_cast<const float4*>(a.gate + static_cast<int64_t>(b) * a.N + n);
    *reinterpret_cast<uint2*>(a.out + o) =
        make_uint2(pack2(fmaf(gv.x, c0, bf_lo(xv.x)), fmaf(gv.y, c1, bf_hi(xv.x))),
                   pack2(fmaf(gv.z, c2, bf_lo(xv.y)), fmaf(gv.w, c3, bf_hi(xv.y))));
  }
}

// --------------------------------------------------------------------- GEMM
// NG groups of 4 waves; group g multiplies the K-steps kt = g (mod NG)
// through its own NS-stage ring, and group 1's accumulators are added into
// group 0's through LDS at the end (NG = 2: two copy streams per CU).
template <int EPI, int NS, int NG>
__global__ __launch_bounds__(kGThreads * NG) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NG * NS * kStageBytes];
  const int tiles_m = (a.M + kBM - 1) / kBM;
  const int tiles = tiles_m * ((a.N + kBN - 1) / kBN);
  const int bid = blockIdx.x;
  const int t = (tiles % 8 == 0) ? (bid % 8) * (tiles / 8) + bid / 8 : bid;
  const int m0 = (t % tiles_m) * kBM, n0 = (t / tiles_m) * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = NG == 1 ? 0 : wave >> 2, w4 = wave & 3;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((TT_LDS uint8_t*)smem));
  TT_LDS const uint8_t* lsm = (TT_LDS const uint8_t*)smem;

  // copies: wave w4 of a group, copy j fills tile rows (4 w4 + j) * 8 .. +8;
  // lane L row r = (4 w4 + j) * 8 + L / 8, LDS slot L % 8 <- k-chunk
  // (L % 8) ^ ((r >> 1) & 7); rows past the matrix end repeat its last row
  // (never stored)
  uint32_t offa[kCopies], offw[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int r = (w4 * kCopies + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int ra = min(r, a.M - 1 - m0), rw = min(r, a.N - 1 - n0);
    offa[j] = static_cast<uint32_t>(ra * a.K * 2 + c * 16);
    offw[j] = static_cast<uint32_t>(rw * a.K * 2 + c * 16);
  }
  const uint16_t* abase = a.a + static_cast<int64_t>(m0) * a.K;
  const uint16_t* wbase = a.w + static_cast<int64_t>(n0) * a.K;
  // the group's i-th step is K-step i * NG + grp, in stage i % NS of its ring
  auto issue = [&](int i) {
    const int kt = i * NG + grp;
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        lds0 + (grp * NS + i % NS) * kStageBytes + w4 * kCopies * 1024);
    const uint32_t lw = la + kTileBytes;
    const uint16_t* ab = abase + kt * kBK;
    const uint16_t* wb = wbase + kt * kBK;
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      dma16s(ab, offa[j], la + j * 1024);
      dma16s(wb, offw[j], lw + j * 1024);
    }
  };

  // operand reads: W rows wn*64 + ns*32 + l%32 (A operand), A rows
  // wm*64 + ms*32 + l%32 (B operand); k-chunk 2 ks + l/32 of step ks
  const int wn = w4 >> 1, wm = w4 & 1;
  const int l32 = lane & 31, half = lane >> 5;
  const int sw = (l32 >> 1) & 7;
  int slot[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) slot[ks] = ((2 * ks + half) ^ sw) * 16;
  const int wrow = (wn * 64 + l32) * 128, arow = (wm * 64 + l32) * 128;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = a.K / kBK;
  const int steps = (KT - grp + NG - 1) / NG;   // this group's K-steps
  const int iters = (KT + NG - 1) / NG;         // the same for every group
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < steps) issue(s0);
  for (int it = 0; it < iters; ++it) {
    // this step's copies (this wave's) are done once at most the later
    // steps' are in flight; the barrier makes every wave's copies visible
    // and frees the stage the copy below overwrites (read in step it-1)
    wait_steps<NS>(min(NS - 2, steps - 1 - it));
    __syncthreads();
    if (it + NS - 1 < steps) issue(it + NS - 1);
    if (it >= steps) continue;           // a group with one step fewer
    TT_LDS const uint8_t* sa = lsm + (grp * NS + it % NS) * kStageBytes;
    TT_LDS const uint8_t* sw_ = sa + kTileBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 wf[2], af[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        wf[i] = *reinterpret_cast<TT_LDS const bf16x8*>(sw_ + wrow + i * 32 * 128 + slot[ks]);
        af[i] = *reinterpret_cast<TT_LDS const bf16x8*>(sa + arow + i * 32 * 128 + slot[ks]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
  }

  if constexpr (NG == 2) {
    // group 1's partial sums into group 0's (64 KB of the ring, conflict
    // free: consecutive lanes, consecutive words)
    TT_LDS float* red = (TT_LDS float*)smem;
    __syncthreads();                     // every wave is done with the ring
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[(((w4 * 2 + i) * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += red[(((w4 * 2 + i) * 2 + j) * 16 + r) * 64 + lane];
  }

  // ---- epilogue: lane holds C[m][n .. n+3] for m = m0 + wm*64 + j*32 + l%32,
  // n = n0 + wn*64 + i*32 + 8 g + 4 (l/32), g < 4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + j * 32 + l32;
    if (m >= a.M) continue;
    const int b = m / a.S;
    if (a.active && !a.active[b]) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + i * 32 + 8 * g + 4 * half;
        if (n >= a.N) continue;
        store4<EPI>(a, m, b, n, acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                    acc[i][j][4 * g + 3]);
      }
  }
}

// 128 x 144 tiles, for shapes whose tile count fits the CUs at this width
// but not at 128 (N = 4608 at M = 1024: 256 tiles instead of 288): two
// groups of 4 waves as in gemm_kernel<EPI, 2, 2>; each wave multiplies all
// 144 W rows of the tile against its 32 A rows with
// v_mfma_f32_16x16x32_bf16 (9 x 2 accumulator tiles of 16 x 16).  A stage
// holds the A tile (16 KB), the W tile (18 KB) and 2 KB that two padding
// copies fill (so that every wave issues 9 copies).
constexpr int kBN144 = 144;
constexpr int kStage144 = 36 * 1024;
constexpr int kCopies144 = 9;            // per wave per stage: 36 copies / 4 waves

template <int EPI>
__global__ __launch_bounds__(2 * kGThreads) void gemm144_kernel(GemmArgs a) {
  constexpr int NS = 2, NG = 2, NT = kBN144 / 16;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NG * NS * kStage144];
  const int tiles_m = (a.M + kBM - 1) / kBM;
  const int tiles = tiles_m * (a.N / kBN144);
  const int bid = blockIdx.x;
  const int t = (tiles % 8 == 0) ? (bid % 8) * (tiles / 8) + bid / 8 : bid;
  const int m0 = (t % tiles_m) * kBM, n0 = (t / tiles_m) * kBN144;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, w4 = wave & 3;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((TT_LDS uint8_t*)smem));
  TT_LDS const uint8_t* lsm = (TT_LDS const uint8_t*)smem;

  // copy q = 9 w4 + j fills stage bytes [q KB, q KB + 1 KB): A rows 8q..
  // (q < 16), W rows 8 (q - 16).. (q < 34), or W rows 0..7 again (padding);
  // lane L: row + L / 8, LDS slot L % 8 <- k-chunk (L % 8) ^ ((row >> 1) & 7)
  uint32_t off[kCopies144];
  bool isw[kCopies144];
#pragma unroll
  for (int j = 0; j < kCopies144; ++j) {
    const int q = w4 * kCopies144 + j;
    isw[j] = q >= 16;
    const int r = (q < 16 ? 8 * q : (q < 34 ? 8 * (q - 16) : 0)) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int rc = q < 16 ? min(r, a.M - 1 - m0) : r;     // N is a multiple of 144
    off[j] = static_cast<uint32_t>(rc * a.K * 2 + c * 16);
  }
  const uint16_t* abase = a.a + static_cast<int64_t>(m0) * a.K;
  const uint16_t* wbase = a.w + static_cast<int64_t>(n0) * a.K;
  auto issue = [&](int i) {
    const int kt = i * NG + grp;
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(
        lds0 + (grp * NS + i % NS) * kStage144 + w4 * kCopies144 * 1024);
#pragma unroll
    for (int j = 0; j < kCopies144; ++j)
      dma16s((isw[j] ? wbase : abase) + kt * kBK, off[j], l0 + j * 1024);
  };

  // operand reads, k-substep ks of 32: W rows 16 nt + l%16 (A operand), A
  // rows 32 w4 + 16 mt + l%16 (B operand), k-chunk 4 ks + l/16
  const int l16 = lane & 15, kq = lane >> 4;
  const int sw = (l16 >> 1) & 7;
  const int slot0 = ((kq) ^ sw) * 16, slot1 = ((4 + kq) ^ sw) * 16;
  const int wrow = l16 * 128, arow = (w4 * 32 + l16) * 128;

  f32x4 acc[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = a.K / kBK;
  const int steps = (KT - grp + NG - 1) / NG;
  const int iters = (KT + NG - 1) / NG;
  if (steps > 0) issue(0);
  for (int it = 0; it < iters; ++it) {
    wait_vmem<0>();                      // this wave's copies of step it
    __syncthreads();                     // everyone's; step it-1's stage is free
    if (it + 1 < steps) issue(it + 1);
    if (it >= steps) continue;
    TT_LDS const uint8_t* sa = lsm + (grp * NS + it % NS) * kStage144;
    TT_LDS const uint8_t* sw_ = sa + kTileBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int slot = ks ? slot1 : slot0;
      bf16x8 af[2], wf[NT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[mt] = *reinterpret_cast<TT_LDS const bf16x8*>(sa + arow + mt * 16 * 128 + slot);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        wf[nt] = *reinterpret_cast<TT_LDS const bf16x8*>(sw_ + wrow + nt * 16 * 128 + slot);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nt], af[mt], acc[nt][mt], 0, 0, 0);
    }
  }

  // group 1's partial sums into group 0's
  TT_LDS float* red = (TT_LDS float*)smem;
  __syncthreads();
  if (grp == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(((w4 * NT + nt) * 2 + mt) * 4 + r) * 64 + lane] = acc[nt][mt][r];
  }
  __syncthreads();
  if (grp == 1) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nt][mt][r] += red[(((w4 * NT + nt) * 2 + mt) * 4 + r) * 64 + lane];

  // ---- epilogue: lane holds C[m][n .. n+3] for m = m0 + 32 w4 + 16 mt + l%16,
  // n = n0 + 16 nt + 4 (l/16)
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int m = m0 + w4 * 32 + mt * 16 + l16;
    if (m >= a.M) continue;
    const int b = m / a.S;
    if (a.active && !a.active[b]) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + nt * 16 + 4 * kq;
      store4<EPI>(a, m, b, n, acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]);
    }
  }
}

}  // namespace

bool ln_supported(int D) { return D >= 8 && D % 8 == 0 && D <= 8192; }

hipError_t launch_ln_modulate(const LnArgs& a, hipStream_t st) {
  const int nch = (a.D + 511) / 512;
  const dim3 grid((a.M + 3) / 4), blk(256);
  switch (nch) {
#define TT_LN(K) \
  case K: hipLaunchKernelGGL(ln_modulate_kernel<K>, grid, blk, 0, st, a); break;
    TT_LN(1) TT_LN(2) TT_LN(3) TT_LN(4) TT_LN(5) TT_LN(6) TT_LN(7) TT_LN(8)
    TT_LN(9) TT_LN(10) TT_LN(11) TT_LN(12) TT_LN(13) TT_LN(14) TT_LN(15) TT_LN(16)
#undef TT_LN
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool gemm_supported(int M, int N, int K) {
  // K in whole 64-steps; 4-column output groups; in-tile byte offsets of
  // the copies fit 32 bits
  return M >= 1 && N >= 4 && N % 4 == 0 && K >= kBK && K % kBK == 0 &&
         static_cast<int64_t>(kBM) * K * 2 < (int64_t(1) << 31);
}

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
  const int tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  // Up to one tile per CU: a 3-stage ring (96 KB of LDS).  More tiles than
  // CUs: a 2-stage ring (64 KB), so that two tiles share a CU and the tiles
  // past the CU count run beside the others instead of in a second round
  // (measured: 288 tiles on 256 CUs take 56 us instead of 80).
  const int cus = device_cus();
  const bool two = tiles > cus;
  const int tiles144 = a.N % kBN144 == 0 ? ((a.M + kBM - 1) / kBM) * (a.N / kBN144) : 0;
  if (two && tiles144 > 0 && tiles144 <= cus) {
    if (epi == kEpiQkv) hipLaunchKernelGGL(gemm144_kernel<kEpiQkv>, dim3(tiles144), dim3(2 * kGThreads), 0, st, a);
    else hipLaunchKernelGGL(gemm144_kernel<kEpiGate>, dim3(tiles144), dim3(2 * kGThreads), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid(tiles);
  if (epi == kEpiQkv) {
    if (two) hipLaunchKernelGGL((gemm_kernel<kEpiQkv, 2, 1>), grid, dim3(kGThreads), 0, st, a);
    else hipLaunchKernelGGL((gemm_kernel<kEpiQkv, 2, 2>), grid, dim3(2 * kGThreads), 0, st, a);
  } else {
    if (two) hipLaunchKernelGGL((gemm_kernel<kEpiGate, 2, 1>), grid, dim3(kGThreads), 0, st, a);
    else hipLaunchKernelGGL((gemm_kernel<kEpiGate, 2, 2>), grid, dim3(2 * kGThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace tt
