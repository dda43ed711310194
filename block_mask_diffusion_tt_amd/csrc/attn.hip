// Per-layer block attention of the denoiser over [context KV ; block KV].
//
// [dothoosh] two-tower mechanism section: inside a block the denoiser
// attends bidirectionally, and causally to the earlier clean blocks; layer i
// of the denoiser talks to layer i of the frozen context tower (whose KV cache
// covers the prompt and the committed tokens).  [modelcard] technical
// features section: bidirectional self-attention in the block plus
// layer-aligned cross-attention to the same layer's context KV; adaLN-single
// scale/shift/gate per timestep.  One softmax spans all keys of a query.
//
// Work decomposition (split-K over the context, flash-decode style):
//   * the R = S*G query rows that share KV head g (S block slots x G query
//     heads of the group) form the M dimension of dense tiles: every K/V
//     tile staged in LDS is used by all of them, so each context byte is
//     read from HBM once per layer;
//   * a unit = (sequence b, KV head g, row block rb, context chunk c); chunk 0
//     also takes the S block keys; units write (max, sum, accumulator)
//     partials that the merge kernel combines in chunk order (deterministic).
//
// bf16 kernel (gfx950 matrix cores, 64-wide waves): 8 waves x 32 rows, one
// workgroup per CU (two waves per SIMD).
//   S^T = K Q'^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 channels
//   straight from the LDS K tile, B = the wave's pre-modulated Q' held in
//   registers), so each lane ends with 16 scores of one row; the online
//   softmax needs only one cross-lane exchange (lanes l and l^32 share rows).
//   O^T += V^T P^T with the same instruction: the scores' accumulator layout
//   is already the B-operand layout of P^T, and the V^T operand comes from
//   the LDS V tile through the transposing ds_read_b64_tr_b16.  Scores are in
//   log2 units (log2(e)/sqrt(d) folded into Q') and relative to a per-row
//   reference mu: the QK^T accumulation starts from -mu, so the exponentials
//   need no subtraction.  mu is only raised when a half-tile exceeds it by
//   more than 8 (values of P stay <= 256), so accumulators are rarely
//   rescaled.  K/V tiles stream HBM -> LDS through the direct copy path in a
//   4-stage ring: three tiles are in flight while one is multiplied.
#include <float.h>
#include <math.h>

#include <type_traits>

#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTK = 64;          // keys per LDS tile
constexpr int kKPad = 8;         // bf16 padding of an LDS K row
constexpr int kVPad = 4;         // bf16 padding of an LDS V^T row
constexpr int kRowsBf16 = 256;   // rows per bf16 workgroup (8 waves x 32)
constexpr int kRowsF32 = 64;     // rows per fp32 workgroup (1 wave, 1 row per lane)
constexpr float kRescaleTh = 8.f;
constexpr float kLog2e = 1.4426950408889634f;

struct KParams {
  int B, S, Hq, Hkv, G, R;
  int rows_per_unit, RB, NC, chunk;
  const uint16_t* q; const uint16_t* kb; const uint16_t* vb;
  const uint16_t* kc; const uint16_t* vc;
  const void* qf; const void* kbf; const void* vbf; const void* kcf; const void* vcf;
  const int64_t* ctx_start; const int32_t* ctx_len; const uint8_t* active;
  const float* shift; const float* scale;
  float qscale;
  void* part_acc; float* part_ml;   // part_acc: fp16 (bf16 kernel) or fp32 (fp32 kernel)
  int causal;                       // block slot s sees block keys 0..s only
  const int64_t* ctx_end;           // non-NULL: append the block's K/V to the cache
  void* kc_out; void* vc_out;
};

struct MParams {
  int B, S, Hq, Hkv, G, R, D;
  int rows_per_unit, RB, NC, chunk;
  const int32_t* ctx_len; const uint8_t* active;
  const float* gate; const void* residual; void* out; float* lse;
  const void* part_acc; const float* part_ml;
};

__device__ __forceinline__ int units_of(int L, int chunk, int NC) {
  int n = (L + chunk - 1) / chunk;
  n = n < 1 ? 1 : n;
  return n > NC ? NC : n;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Decode the unit of this workgroup; false when it has nothing to do.
struct Unit {
  int b, g, rb, c, nunits;
  int k_beg, k_end;   // context keys of this unit
  bool has_blk;
};

__device__ __forceinline__ bool decode_unit(int u, int Hkv, int RB, int NC, int chunk,
                                            const int32_t* ctx_len, const uint8_t* active,
                                            Unit& un) {
  un.c = u % NC;
  int t = u / NC;
  un.rb = t % RB;
  t /= RB;
  un.g = t % Hkv;
  un.b = t / Hkv;
  if (active && !active[un.b]) return false;
  const int L = ctx_len[un.b];
  un.nunits = units_of(L, chunk, NC);
  if (un.c >= un.nunits) return false;
  un.k_beg = un.c * chunk;
  un.k_end = (un.c == un.nunits - 1) ? L : (un.c + 1) * chunk;
  if (un.k_end < un.k_beg) un.k_end = un.k_beg;  // L == 0
  un.has_blk = (un.c == 0);
  return true;
}

// The context tower's cache append, done by the unit that owns the block
// keys of (b, g): block rows s < S of KV head g are copied to cache rows
// ctx_start[b] + ctx_len[b] + s when the sequence's reserved region
// [ctx_start[b], ctx_end[b]) has room for them.  No unit reads those rows
// (every unit of b reads context rows below ctx_len[b]), so the copies need
// no ordering with the attention.  16-byte pieces, all threads of the
// workgroup.
__device__ __forceinline__ void append_block_kv(const KParams& p, const Unit& un, int D, int esize) {
  if (!p.ctx_end || !un.has_blk || un.rb != 0) return;
  const int64_t st = p.ctx_start[un.b];
  const int64_t L = p.ctx_len[un.b];
  if (L + p.S > p.ctx_end[un.b] - st) return;
  const int per_row = D * esize / 16;
  const int n = p.S * per_row;
  const int64_t row_bytes = static_cast<int64_t>(p.Hkv) * D * esize;
  const char* kb = static_cast<const char*>(p.kbf) + (static_cast<int64_t>(un.b) * p.S * p.Hkv + un.g) * D * esize;
  const char* vb = static_cast<const char*>(p.vbf) + (static_cast<int64_t>(un.b) * p.S * p.Hkv + un.g) * D * esize;
  char* kd = static_cast<char*>(p.kc_out) + ((st + L) * p.Hkv + un.g) * D * esize;
  char* vd = static_cast<char*>(p.vc_out) + ((st + L) * p.Hkv + un.g) * D * esize;
  for (int i = threadIdx.x; i < 2 * n; i += blockDim.x) {
    const int j = i < n ? i : i - n;
    const int64_t off = (j / per_row) * row_bytes + (j % per_row) * 16;
    if (i < n)
      *reinterpret_cast<uint4*>(kd + off) = *reinterpret_cast<const uint4*>(kb + off);
    else
      *reinterpret_cast<uint4*>(vd + off) = *reinterpret_cast<const uint4*>(vb + off);
  }
}

// ------------------------------------------------------------------ bf16
#define TT_LDS __attribute__((address_space(3)))
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16-byte global -> LDS copy through the direct path: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16).  Written in asm because the compiler would
// otherwise wait for every such copy in flight before any LDS read (it cannot
// tell the pipeline stages apart); the stage waits below are explicit.  The
// instruction has no register result.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds) : "memory");
}

// The same copy from a wave-uniform base plus a per-lane byte offset (the
// SGPR-base form: no per-copy address arithmetic), marked non-temporal: the
// context K/V is read once per layer, so the caches need not keep it.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(off), "s"(base), "s"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// max / sum of a value over lanes l and l^32 (the two halves of a wave)
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// e[r0..r0+7] rounded to bf16 (round to nearest even), packed in order
__device__ __forceinline__ bf16x8 pack_bf16(const float (&e)[16], int r0) {
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {static_cast<__bf16>(e[r0 + 2 * i]), static_cast<__bf16>(e[r0 + 2 * i + 1])};
    pk[i] = __builtin_bit_cast(uint32_t, pr);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
}

// Instruction interleaving requests for the machine scheduler: groups of
// `n` instructions of one class, in the order requested (class masks of
// the scheduler: 0x8 matrix products, 0x402 vector ALU incl. transcendental,
// 0x100 LDS reads).
constexpr int kSchedMfma = 0x8, kSchedValu = 0x402, kSchedLdsRead = 0x100;
#define TT_SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

// Keeps a value's computation before this point: an empty asm that reads and
// "writes" the register, so the compiler cannot sink the arithmetic that
// produces it into a later basic block.
#define TT_PIN(x) asm volatile("" : "+v"(x))

template <int D>
struct Bf16Cfg {
  static constexpr int CH = D / 8;                 // 16-byte chunks per key row
  static constexpr int TILE = 64 * D * 2;          // bytes of one K (or V) tile of 64 keys
  static constexpr int NST = 4;                    // pipeline stages
  static constexpr int VREG = NST * TILE;          // V tiles follow the NST K tiles
  static constexpr int CPT = 64 * CH / 512;        // copies per thread per tile tensor
  static constexpr int SMEM = 2 * NST * TILE;
};

// LDS tile layouts (16-byte slots).  K: slot = (key/16)*16*CH + c*16 + key%16
// (chunk-major inside groups of 16 keys), so the 16 lanes reading one chunk of
// 16 consecutive keys hit 16 different bank groups and every chunk offset is
// an immediate.  V: slot = (key/4)*4*CH + c*4 + key%4 (4 keys interleaved per
// chunk), so the transpose reads of 4 keys x 4 chunks x 2 halves by 32 lanes
// hit all 64 banks once, and a 64-slot copy is 4 whole key rows.
template <int D>
__device__ __forceinline__ int kslot(int key, int c) {
  return (key >> 4) * 16 * (D / 8) + c * 16 + (key & 15);
}
template <int D>
__device__ __forceinline__ int vslot(int key, int c) {
  return (key >> 2) * 4 * (D / 8) + c * 4 + (key & 3);
}


template <int D>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(KParams p) {
  using C = Bf16Cfg<D>;
  constexpr int KSTEPS = D / 16;   // MFMA k-steps of QK^T
  constexpr int DT = D / 32;       // 32-channel tiles of the output
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::SMEM];

  Unit un;
  if (!decode_unit(blockIdx.x, p.Hkv, p.RB, p.NC, p.chunk, p.ctx_len, p.active, un)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const int64_t kstride = static_cast<int64_t>(p.Hkv) * D;
  TT_LDS uint8_t* const lsm = (TT_LDS uint8_t*)(smem);  // address-space cast
  append_block_kv(p, un, D, 2);
  // block keys visible to this lane's row: all S, or slots 0..s when causal
  // (rows past R take all S, so every row has a finite maximum)
  int blk_valid = p.S;
  if (p.causal) {
    const int row = un.rb * kRowsBf16 + wave * 32 + l32;
    blk_valid = row < p.R ? row / p.G + 1 : p.S;
  }
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lsm));

  // ---- Q' = (q * (1 + scale) + shift) * log2(e)/sqrt(d), rounded to bf16;
  // this wave's 32 rows, lane l32 holding row wave*32 + l32
  bf16x8 qf[KSTEPS];
  {
    const int row = un.rb * kRowsBf16 + wave * 32 + l32;
    const bool valid = row < p.R;
    const int s = valid ? row / p.G : 0;
    const int h = un.g * p.G + (valid ? row % p.G : 0);
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(un.b) * p.S + s) * p.Hq + h) * D;
    const float* sc = p.scale ? p.scale + (static_cast<int64_t>(un.b) * p.Hq + h) * D : nullptr;
    const float* sh = p.shift ? p.shift + (static_cast<int64_t>(un.b) * p.Hq + h) * D : nullptr;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int d0 = kk * 16 + half * 8;
      float v[8];
      const uint4 w = valid ? *reinterpret_cast<const uint4*>(qrow + d0) : make_uint4(0, 0, 0, 0);
      v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
      v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
      v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xffff0000u);
      v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xffff0000u);
      if (sc && valid) {
        const float4 a = *reinterpret_cast<const float4*>(sc + d0);
        const float4 b = *reinterpret_cast<const float4*>(sc + d0 + 4);
        v[0] *= 1.f + a.x; v[1] *= 1.f + a.y; v[2] *= 1.f + a.z; v[3] *= 1.f + a.w;
        v[4] *= 1.f + b.x; v[5] *= 1.f + b.y; v[6] *= 1.f + b.z; v[7] *= 1.f + b.w;
      }
      if (sh && valid) {
        const float4 a = *reinterpret_cast<const float4*>(sh + d0);
        const float4 b = *reinterpret_cast<const float4*>(sh + d0 + 4);
        v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
        v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[kk][i] = static_cast<__bf16>(v[i] * p.qscale);
    }
  }

  // ---- tiles: the block's S keys first (chunk 0), then 64-key context tiles
  const int n_ctx_tiles = (un.k_end - un.k_beg + kTK - 1) / kTK;
  const int n_tiles = (un.has_blk ? 1 : 0) + n_ctx_tiles;
  const int64_t ctx0 = p.ctx_start[un.b];
  auto tile_valid = [&](int t) {
    return (un.has_blk && t == 0) ? blk_valid
                                  : min(kTK, un.k_end - (un.k_beg + (t - (un.has_blk ? 1 : 0)) * kTK));
  };
  // Copy m (0 <= m < CH) of a tile tensor fills 16-byte slots [64m, 64m+64):
  // for K, 16 keys x 4 chunks (key 16*(m/(CH/4)) + lane%16, chunk
  // 4*(m%(CH/4)) + lane/16); for V, 64 consecutive slots of the
  // 4-key-interleaved layout (whole key rows).  Wave w issues copies
  // m = w*CPT .. w*CPT+CPT-1.  Full tiles use precomputed byte offsets from a
  // wave-uniform tile base; a tile with fewer than 64 keys repeats its last
  // key (finite values whose scores are masked to -inf).  K tiles of the NST
  // stages come first, then V tiles.
  auto kkey_of = [&](int m) { return 16 * (m / (C::CH / 4)) + (lane & 15); };
  auto kch_of = [&](int m) { return 4 * (m % (C::CH / 4)) + (lane >> 4); };
  auto vkey_of = [&](int m) { const int s0 = 64 * m + lane; return 4 * (s0 / (4 * C::CH)) + (s0 & 3); };
  auto vch_of = [&](int m) { const int s0 = 64 * m + lane; return (s0 % (4 * C::CH)) >> 2; };
  uint32_t koff[C::CPT], voff[C::CPT];
#pragma unroll
  for (int j = 0; j < C::CPT; ++j) {
    const int m = wave * C::CPT + j;
    koff[j] = static_cast<uint32_t>((kkey_of(m) * kstride + kch_of(m) * 8) * 2);
    voff[j] = static_cast<uint32_t>((vkey_of(m) * kstride + vch_of(m) * 8) * 2);
  }
  auto issue = [&](int t) {
    const int stage = t % C::NST;
    const uint16_t* kp;
    const uint16_t* vp;
    int nv;
    if (un.has_blk && t == 0) {
      const int64_t off = (static_cast<int64_t>(un.b) * p.S * p.Hkv + un.g) * D;
      kp = p.kb + off;
      vp = p.vb + off;
      nv = p.S;
    } else {
      const int key0 = un.k_beg + (t - (un.has_blk ? 1 : 0)) * kTK;
      const int64_t off = ((ctx0 + key0) * p.Hkv + un.g) * D;
      kp = p.kc + off;
      vp = p.vc + off;
      nv = min(kTK, un.k_end - key0);
    }
    const uint32_t kl = __builtin_amdgcn_readfirstlane(lds0 + stage * C::TILE + wave * C::CPT * 1024);
    const uint32_t vl = __builtin_amdgcn_readfirstlane(lds0 + C::VREG + stage * C::TILE + wave * C::CPT * 1024);
    if (nv == kTK) {
#pragma unroll
      for (int j = 0; j < C::CPT; ++j) {
        dma16s(kp, koff[j], kl + j * 1024);
        dma16s(vp, voff[j], vl + j * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::CPT; ++j) {
        const int m = wave * C::CPT + j;
        const uint32_t ko = static_cast<uint32_t>((min(kkey_of(m), nv - 1) * kstride + kch_of(m) * 8) * 2);
        const uint32_t vo = static_cast<uint32_t>((min(vkey_of(m), nv - 1) * kstride + vch_of(m) * 8) * 2);
        dma16s(kp, ko, kl + j * 1024);
        dma16s(vp, vo, vl + j * 1024);
      }
    }
  };

  // per-lane operand bases (bytes within a stage): K chunk 2kk+half of key
  // kt*32 + l32 is at kbase + kt*32*CH*16 + kk*2*16*16; the V^T transpose read
  // of channel tile dt, 16-key step ks, second 4-key group r2 is at vbase +
  // (kt*8 + ks*4 + r2*2)*4*CH*16 + dt*4*4*16.
  const int kbase = kslot<D>(l32, half) * 16;
  const int vlo = 2 * (grp & 1) + ((li & 3) >> 1);
  const int vbase = C::VREG + vslot<D>(4 * half + (li >> 2), vlo) * 16 + ((li & 1) << 3);

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  // Scores are kept relative to the row's running reference mu: the QK^T
  // accumulation starts from -mu (negmu, all 16 entries of a lane belong to
  // one row), so no subtraction is needed before the exponentials.
  float mu = 0.f;
  float lsum = 0.f;
  f32x16 negmu;
#pragma unroll
  for (int r = 0; r < 16; ++r) negmu[r] = 0.f;

  // K operands of half kt of the tile in `stage` (A of S^T = K Q'^T)
  auto kload = [&](int stage, int kt, bf16x8 (&ko)[KSTEPS]) {
    TT_LDS const uint8_t* kb = lsm + stage * C::TILE + kt * 32 * C::CH * 16 + kbase;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      ko[kk] = *reinterpret_cast<TT_LDS const bf16x8*>(kb + kk * 2 * 16 * 16);
  };
  // S^T of 32 keys x this wave's 32 rows
  auto qk = [&](const bf16x8 (&ko)[KSTEPS], f32x16& sc) {
    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ko[0], qf[0], negmu, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < KSTEPS; ++kk)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ko[kk], qf[kk], sc, 0, 0, 0);
  };
  // V^T operands of k-step ks (keys 16ks..16ks+15) of half kt (A of
  // O^T += V^T P^T), two transpose reads each
  auto vload = [&](int stage, int kt, int ks, bf16x8 (&vo)[2][DT]) {
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    TT_LDS uint8_t* vb = lsm + stage * C::TILE + kt * 8 * 4 * C::CH * 16 + vbase + ks * 4 * 4 * C::CH * 16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      TT_LDS uint8_t* a = vb + dt * 4 * 4 * 16;
      const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<TT_LDS v4i16*>(a));
      const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<TT_LDS v4i16*>(a + 2 * 4 * C::CH * 16));
      const v8i16 w8 = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
      vo[ks][dt] = __builtin_bit_cast(bf16x8, w8);
    }
  };
  auto pv = [&](const bf16x8 (&vo)[2][DT], const bf16x8 (&pb)[2], int ks) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vo[ks][dt], pb[ks], acc[dt], 0, 0, 0);
  };
  // mask keys at or past nvalid in half kt, return the maximum of this
  // lane's 16 scores (lanes l and l^32 hold the two halves of a row)
  auto rowmax = [&](f32x16& sc, int kt, int nvalid) {
    if (__builtin_expect(nvalid < kt * 32 + 32, 0)) {
      // key of accumulator r is kt*32 + 4*half + 8*(r/4) + r%4
      const int lim = nvalid - kt * 32 - 4 * ((static_cast<int>(threadIdx.x) >> 5) & 1);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
    }
    float m = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m = fmaxf(m, fmaxf(sc[r], sc[r + 1]));
    return m;
  };
  auto rowmax_full = [&](const f32x16& sc) {
    float m = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m = fmaxf(m, fmaxf(sc[r], sc[r + 1]));
    return m;
  };
  // raise the reference only when a half-tile exceeds it by more than 2^8
  // (scores are relative to mu): the lane maxima decide, and only then are
  // the two halves of each row combined, so both lanes of a row move mu
  // together; sc is shifted to the new reference
  auto rescale = [&](float lmax, f32x16& sc) {
    if (__any(lmax > kRescaleTh)) {
      const float up = fmaxf(xhalf_max(lmax), 0.f);
      const float alpha = __builtin_amdgcn_exp2f(-up);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      mu += up;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] -= up;
        negmu[r] = -mu;
      }
    }
  };
  // P = 2^S (scores relative to mu) rounded to bf16, the B operand of P^T,
  // in two parts: exponentials 0..kExpA-1 and the k-step-0 operand pb[0]
  // (overlapped with the QK^T products), then the rest and pb[1]
  // (overlapped with the first PV^T products).  The row sum adds the fp32
  // values in two chains of plain adds: the dot-product instruction would
  // serialize with the matrix products.
  constexpr int kExpA = 10;
  auto softmax_a = [&](const f32x16& sc, float (&e)[16], bf16x8 (&pb)[2]) {
#pragma unroll
    for (int r = 0; r < kExpA; ++r) e[r] = __builtin_amdgcn_exp2f(sc[r]);
    pb[0] = pack_bf16(e, 0);
  };
  auto softmax_b = [&](const f32x16& sc, float (&e)[16], bf16x8 (&pb)[2]) {
#pragma unroll
    for (int r = kExpA; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(sc[r]);
    pb[1] = pack_bf16(e, 8);
  };
  auto row_sum = [&](const float (&e)[16]) {
    float s0 = e[0], s1 = e[1];
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      s0 += e[r];
      s1 += e[r + 1];
    }
    lsum += s0 + s1;
  };
  constexpr int LD = 2 * C::CPT;  // copies per thread per tile
  // wait until this thread's copies of tile t have landed (`later` tiles
  // issued after it may still be in flight), then make everyone's visible
  auto wait_tile = [&](int later) {
    if (later >= 1) wait_vmem<LD>();
    else wait_vmem<0>();
    __syncthreads();
  };

  // Pipeline (per wave; tile t in stage t % 4, halves h = 0, 1).  Each
  // half-tile runs three phases, each a run of matrix products with the
  // vector work that does not feed them interleaved:
  //   1. S(next) = QK (8 products)    with exponentials 0..9 of P(h), pb[0]
  //   2. O += PV(h) k-step 0 (4)      with exponentials 10..15, pb[1]; the
  //                                   K operands of the next QK are read
  //   3. O += PV(h) k-step 1 (4)      with the row sum of P(h) and the row
  //                                   maximum of S(next); the V^T operands of
  //                                   the next half's k-step 0 are read
  // where S(next) is S(t,1) in half 0 and S(t+1,0) in half 1.  At the start
  // of tile t the workgroup waits until tile t+1 is visible and issues the
  // copies of tile t+3 into the stage of tile t-1, so every LDS operand read
  // has a full phase or more before its products.  Only the first tile (the
  // block's S keys) and the last context tile can hold fewer than 64 keys;
  // the steps that touch them mask scores, the others do not.
  const int pre = n_tiles < C::NST - 1 ? n_tiles : C::NST - 1;
  for (int t = 0; t < pre; ++t) issue(t);
  wait_tile(n_tiles > 2 ? 1 : (n_tiles - 1));   // tile 0 (tiles 1..2 may fly)
  f32x16 sA, sB;
  bf16x8 pb[2];
  bf16x8 ko[KSTEPS];
  bf16x8 vo[2][DT];
  kload(0, 0, ko);
  qk(ko, sA);
  kload(0, 1, ko);
  vload(0, 0, 0, vo);
  float tmax = xhalf_max(rowmax(sA, 0, tile_valid(0)));
  // the first half-tile sets the reference to its row maximum (finite: the
  // first half of a unit's first tile always holds a valid key)
  mu = tmax;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sA[r] -= tmax;
    negmu[r] = -mu;
  }
  tmax = 0.f;
  // interleaving of the three phases (one product, then vector or LDS work)
  auto sched_phase1 = [&]() {
#pragma unroll
    for (int i = 0; i < KSTEPS - 1; ++i) {
      TT_SCHED_GROUP(kSchedMfma, 1);
      TT_SCHED_GROUP(kSchedValu, 2);
    }
    TT_SCHED_GROUP(kSchedMfma, 1);
  };
  auto sched_phase2 = [&](bool kreads) {
#pragma unroll
    for (int i = 0; i < DT; ++i) {
      TT_SCHED_GROUP(kSchedMfma, 1);
      TT_SCHED_GROUP(kSchedValu, 3);
      if (kreads) TT_SCHED_GROUP(kSchedLdsRead, KSTEPS / DT);
    }
  };
  auto sched_phase3 = [&]() {
#pragma unroll
    for (int i = 0; i < DT; ++i) {
      TT_SCHED_GROUP(kSchedMfma, 1);
      TT_SCHED_GROUP(kSchedValu, 6);
    }
  };
  auto tile_step = [&](int t, auto more_c, auto mask_c) {
    constexpr bool MORE = decltype(more_c)::value;   // a tile t+1 follows
    constexpr bool MASK = decltype(mask_c)::value;   // tile t or t+1 may be partial
    const int st = t % C::NST;
    const int st1 = (t + 1) % C::NST;
    if (MORE) {
      wait_tile(t + 2 < n_tiles ? 1 : 0);          // tile t+1 visible
      if (t + C::NST - 1 < n_tiles) issue(t + C::NST - 1);
    }
    float e[16];
    // ---- half 0: P(t,0) from sA; S(t,1) into sB
    vload(st, 0, 1, vo);
    rescale(tmax, sA);
    softmax_a(sA, e, pb);
    qk(ko, sB);                                    // K(t,1)
    sched_phase1();
    softmax_b(sA, e, pb);
    pv(vo, pb, 0);
    if (MORE) kload(st1, 0, ko);                   // K(t+1,0)
    sched_phase2(MORE);
    pv(vo, pb, 1);
    vload(st, 1, 0, vo);
    row_sum(e);
    tmax = MASK ? rowmax(sB, 1, tile_valid(t)) : rowmax_full(sB);
    sched_phase3();
    TT_PIN(tmax);
    TT_PIN(lsum);
    // ---- half 1: P(t,1) from sB; S(t+1,0) into sA
    vload(st, 1, 1, vo);
    rescale(tmax, sB);
    softmax_a(sB, e, pb);
    if (MORE) {
      qk(ko, sA);                                  // K(t+1,0)
      sched_phase1();
    }
    softmax_b(sB, e, pb);
    pv(vo, pb, 0);
    if (MORE) kload(st1, 1, ko);                   // K(t+1,1)
    sched_phase2(MORE);
    pv(vo, pb, 1);
    if (MORE) {
      vload(st1, 0, 0, vo);                        // V(t+1,0), k-step 0
      row_sum(e);
      tmax = MASK ? rowmax(sA, 0, tile_valid(t + 1)) : rowmax_full(sA);
      sched_phase3();
      TT_PIN(tmax);
    } else {
      row_sum(e);
    }
    TT_PIN(lsum);
  };
  if (n_tiles >= 2) tile_step(0, std::true_type{}, std::true_type{});
  for (int t = 1; t + 2 < n_tiles; ++t) tile_step(t, std::true_type{}, std::false_type{});
  if (n_tiles >= 3) tile_step(n_tiles - 2, std::true_type{}, std::true_type{});
  tile_step(n_tiles - 1, std::false_type{}, std::true_type{});

  // ---- partials: (max, sum) per row and the unnormalised accumulator
  const int64_t u = blockIdx.x;
  const float ltot = xhalf_sum(lsum);
  const int rl = wave * 32 + l32;
  if (un.rb * kRowsBf16 + rl >= p.R) return;
  // o = acc / l in fp16, scaled by 2^-k so the row's largest |o| lands in
  // [2^14, 2^15): full fp16 precision (2^-11 relative) whatever the scale of
  // V, no overflow; (m, l, k) in fp32.  k stays in [-100, 127] so that 2^-k
  // / l and the merge's weight 2^k w l are finite, normal fp32 numbers.
  const float inv = 1.f / ltot;
  float amax = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[dt][r]));
  int ex;
  frexpf(xhalf_max(amax) * inv, &ex);
  const int k = min(max(ex - 15, -100), 127);
  const float sc = ldexpf(inv, -k);
  if (half == 0)
    *reinterpret_cast<float4*>(p.part_ml + (u * kRowsBf16 + rl) * 4) =
        make_float4(mu, ltot, static_cast<float>(k), 0.f);
  uint16_t* dst = static_cast<uint16_t*>(p.part_acc) + (u * kRowsBf16 + rl) * D;
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half4 h = {static_cast<_Float16>(acc[dt][4 * j] * sc), static_cast<_Float16>(acc[dt][4 * j + 1] * sc),
                       static_cast<_Float16>(acc[dt][4 * j + 2] * sc), static_cast<_Float16>(acc[dt][4 * j + 3] * sc)};
      *reinterpret_cast<uint2*>(dst + dt * 32 + 8 * j + 4 * half) = __builtin_bit_cast(uint2, h);
    }
}

// ------------------------------------------------------------------ fp32
// Full-precision path: one lane per query row, fp32 throughout, exact running
// max.  Used for fp32 storage (small problems and precision checks).
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(KParams p) {
  constexpr int TKF = 16;
  __shared__ float qs[kRowsF32][D + 1];
  __shared__ float ks[TKF][D];
  __shared__ float vs[TKF][D];
  Unit un;
  if (!decode_unit(blockIdx.x, p.Hkv, p.RB, p.NC, p.chunk, p.ctx_len, p.active, un)) return;
  const int tid = threadIdx.x;
  const float* q = static_cast<const float*>(p.qf);
  const float* kb = static_cast<const float*>(p.kbf);
  const float* vb = static_cast<const float*>(p.vbf);
  const float* kc = static_cast<const float*>(p.kcf);
  const float* vc = static_cast<const float*>(p.vcf);
  const int64_t kstride = static_cast<int64_t>(p.Hkv) * D;
  const int row = un.rb * kRowsF32 + tid;
  const bool valid = row < p.R;
  append_block_kv(p, un, D, 4);
  // block keys visible to this row: all S, or slots 0..s when causal
  const int blk_valid = (p.causal && valid) ? row / p.G + 1 : p.S;
  {
    const int s = valid ? row / p.G : 0;
    const int h = un.g * p.G + (valid ? row % p.G : 0);
    const float* qrow = q + ((static_cast<int64_t>(un.b) * p.S + s) * p.Hq + h) * D;
    const float* sc = p.scale ? p.scale + (static_cast<int64_t>(un.b) * p.Hq + h) * D : nullptr;
    const float* sh = p.shift ? p.shift + (static_cast<int64_t>(un.b) * p.Hq + h) * D : nullptr;
    for (int dd = 0; dd < D; ++dd) {
      float v = valid ? qrow[dd] : 0.f;
      if (valid && sc) v = v * (1.f + sc[dd]);
      if (valid && sh) v = v + sh[dd];
      qs[tid][dd] = v * p.qscale;
    }
  }
  float acc[D];
#pragma unroll
  for (int dd = 0; dd < D; ++dd) acc[dd] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int64_t ctx0 = p.ctx_start[un.b];
  const int n_blk_tiles = un.has_blk ? (p.S + TKF - 1) / TKF : 0;
  const int n_ctx_tiles = (un.k_end - un.k_beg + TKF - 1) / TKF;
  const int n_tiles = n_blk_tiles + n_ctx_tiles;
  for (int t = 0; t < n_tiles; ++t) {
    const float* kp;
    const float* vp;
    int nv;
    if (t < n_blk_tiles) {
      const int64_t off = ((static_cast<int64_t>(un.b) * p.S + t * TKF) * p.Hkv + un.g) * D;
      kp = kb + off;
      vp = vb + off;
      nv = min(TKF, p.S - t * TKF);
    } else {
      const int key0 = un.k_beg + (t - n_blk_tiles) * TKF;
      const int64_t off = ((ctx0 + key0) * p.Hkv + un.g) * D;
      kp = kc + off;
      vp = vc + off;
      nv = min(TKF, un.k_end - key0);
    }
    __syncthreads();
    for (int idx = tid; idx < TKF * D; idx += 64) {
      const int key = idx / D, dd = idx % D;
      ks[key][dd] = key < nv ? kp[key * kstride + dd] : 0.f;
      vs[key][dd] = key < nv ? vp[key * kstride + dd] : 0.f;
    }
    __syncthreads();
    const int nk = t < n_blk_tiles ? min(nv, blk_valid - t * TKF) : nv;
    for (int key = 0; key < nk; ++key) {
      float s = 0.f;
#pragma unroll 8
      for (int dd = 0; dd < D; ++dd) s = fmaf(qs[tid][dd], ks[key][dd], s);
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float pr = exp2f(s - mn);
      l = l * alpha + pr;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) acc[dd] = fmaf(pr, vs[key][dd], acc[dd] * alpha);
      m = mn;
    }
  }
  if (!valid) return;
  const int64_t u = blockIdx.x;
  *reinterpret_cast<float4*>(p.part_ml + (u * kRowsF32 + tid) * 4) = make_float4(m, l, 0.f, 0.f);
  float* dst = static_cast<float*>(p.part_acc) + (u * kRowsF32 + tid) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int dd = 0; dd < D; ++dd) dst[dd] = acc[dd] * inv;
}

// ------------------------------------------------------------------ merge
// o = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, combined in chunk
// order; lse = ln2 * (M + log2 sum); out = residual + gate * o.
template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* dst, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = {static_cast<__bf16>(a), static_cast<__bf16>(b), static_cast<__bf16>(c),
              static_cast<__bf16>(d)};
  *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, v);
}

template <typename OutT>
__device__ __forceinline__ void load4(const OutT* src, float (&v)[4]);

template <>
__device__ __forceinline__ void load4<float>(const float* src, float (&v)[4]) {
  const float4 x = *reinterpret_cast<const float4*>(src);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}

template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* src, float (&v)[4]) {
  const uint2 x = *reinterpret_cast<const uint2*>(src);
  v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xffff0000u);
  v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xffff0000u);
}

// N consecutive partial values from element offset `off`: fp16 partials
// (bf16 output) or fp32 partials (fp32 output), in 16-byte loads.
template <typename OutT, int N>
__device__ __forceinline__ void load_part(const void* part, int64_t off, float (&a)[N]);

template <>
__device__ __forceinline__ void load_part<float, 8>(const void* part, int64_t off, float (&a)[8]) {
  const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(part) + off);
  const float4 x = src[0], y = src[1];
  a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
  a[4] = y.x; a[5] = y.y; a[6] = y.z; a[7] = y.w;
}

template <>
__device__ __forceinline__ void load_part<uint16_t, 8>(const void* part, int64_t off, float (&a)[8]) {
  typedef _Float16 half8 __attribute__((ext_vector_type(8)));
  const half8 h = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(part) + off));
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = static_cast<float>(h[i]);
}

// Each thread owns kMergeQuads 4-channel quads of one row (16-byte loads);
// a workgroup covers 256 / (D / (4 kMergeQuads)) rows of one (sequence, KV
// head, row block) group.  Two quads per thread measured fastest (1, 2, 4
// and 8 tried at the headline shape: 10.1, 8.6, 10.1, 13.0 us).
constexpr int kMergeQuads = 2;
template <int D>
constexpr int merge_rows_per_wg() { return 256 / (D / (4 * kMergeQuads)); }

template <typename OutT, int D>
__global__ __launch_bounds__(256) void merge_kernel(MParams p) {
  constexpr int CPT = 4 * kMergeQuads;   // channels per thread
  constexpr int Q = kMergeQuads;         // 16-byte loads per thread per chunk
  constexpr int TPR = D / CPT;           // threads per row
  const int grp = blockIdx.y;  // (b, g, rb)
  const int rb = grp % p.RB;
  const int g = (grp / p.RB) % p.Hkv;
  const int b = grp / (p.RB * p.Hkv);
  if (p.active && !p.active[b]) return;
  const int rl = blockIdx.x * merge_rows_per_wg<D>() + threadIdx.x / TPR;
  const int c0 = (threadIdx.x % TPR) * CPT;
  if (rl >= p.rows_per_unit) return;
  const int row = rb * p.rows_per_unit + rl;
  if (row >= p.R) return;
  const int n = units_of(p.ctx_len[b], p.chunk, p.NC);
  const int64_t u0 = static_cast<int64_t>(grp) * p.NC;
  // chunk c contributes w_c l_c o_c with w_c = 2^(m_c - M); its stored
  // partial is o_c 2^-k_c (fp16 for bf16 output, fp32 for fp32 output)
  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, p.part_ml[((u0 + c) * p.rows_per_unit + rl) * 4]);
  float L = 0.f;
  float o[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) o[i] = 0.f;
  for (int c = 0; c < n; ++c) {
    const int64_t base = (u0 + c) * p.rows_per_unit + rl;
    const float4 ml = *reinterpret_cast<const float4*>(p.part_ml + base * 4);
    const float wl = exp2f(ml.x - M) * ml.y;
    L += wl;
    const float coef = ldexpf(wl, static_cast<int>(ml.z));
    float a[CPT];
    load_part<OutT, CPT>(p.part_acc, base * D + c0, a);
#pragma unroll
    for (int i = 0; i < CPT; ++i) o[i] = fmaf(coef, a[i], o[i]);
  }
  const float inv = 1.f / L;
  const int s = row / p.G, h = g * p.G + row % p.G;
  const int64_t orow = (static_cast<int64_t>(b) * p.S + s) * p.Hq + h;
  const float* gp = p.gate ? p.gate + (static_cast<int64_t>(b) * p.Hq + h) * D + c0 : nullptr;
  const OutT* rp = p.residual ? static_cast<const OutT*>(p.residual) + orow * D + c0 : nullptr;
  OutT* op = static_cast<OutT*>(p.out) + orow * D + c0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    float v[4] = {o[4 * q] * inv, o[4 * q + 1] * inv, o[4 * q + 2] * inv, o[4 * q + 3] * inv};
    if (gp) {
      const float4 gv = *reinterpret_cast<const float4*>(gp + 4 * q);
      v[0] *= gv.x; v[1] *= gv.y; v[2] *= gv.z; v[3] *= gv.w;
    }
    if (rp) {
      float r[4];
      load4<OutT>(rp + 4 * q, r);
      v[0] += r[0]; v[1] += r[1]; v[2] += r[2]; v[3] += r[3];
    }
    store4<OutT>(op + 4 * q, v[0], v[1], v[2], v[3]);
  }
  if (p.lse && c0 == 0) p.lse[orow] = 0.6931471805599453f * (M + log2f(L));
}

}  // namespace

AttnPlan attn_plan(int B, int S, int Hq, int Hkv, int d, int dtype, int max_ctx_len) {
  AttnPlan pl{};
  const int G = Hq / Hkv;
  pl.rows = S * G;
  pl.rows_per_unit = dtype == 0 ? kRowsBf16 : kRowsF32;
  pl.row_blocks = static_cast<int>(ceil_div(pl.rows, pl.rows_per_unit));
  const int64_t groups = static_cast<int64_t>(B) * Hkv * pl.row_blocks;
  const int64_t want = ceil_div(kNumCUs, groups);
  int64_t chunk = max_ctx_len > 0 ? ceil_div(max_ctx_len, want < 1 ? 1 : want) : kTK;
  chunk = static_cast<int64_t>(align_up(static_cast<size_t>(chunk), kTK));
  if (chunk < kTK) chunk = kTK;
  pl.chunk = static_cast<int>(chunk);
  int64_t nc = max_ctx_len > 0 ? ceil_div(max_ctx_len, chunk) : 1;
  pl.n_chunks = static_cast<int>(nc < 1 ? 1 : nc);
  const int64_t units = groups * pl.n_chunks;
  pl.groups = groups;
  const size_t part_elt = dtype == 0 ? 2 : 4;   // fp16 partials for bf16, fp32 for fp32
  pl.part_acc_bytes = align_up(static_cast<size_t>(units) * pl.rows_per_unit * d * part_elt, 256);
  pl.part_ml_bytes = align_up(static_cast<size_t>(units) * pl.rows_per_unit * 4 * sizeof(float), 256);
  pl.total_bytes = pl.part_acc_bytes + pl.part_ml_bytes;
  return pl;
}

hipError_t launch_block_attn(const AttnArgs& a, const AttnPlan& pl, void* ws, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  KParams kp{};
  kp.B = a.B; kp.S = a.S; kp.Hq = a.Hq; kp.Hkv = a.Hkv; kp.G = G; kp.R = pl.rows;
  kp.rows_per_unit = pl.rows_per_unit; kp.RB = pl.row_blocks; kp.NC = pl.n_chunks;
  kp.chunk = pl.chunk;
  kp.q = static_cast<const uint16_t*>(a.q); kp.kb = static_cast<const uint16_t*>(a.kb);
  kp.vb = static_cast<const uint16_t*>(a.vb); kp.kc = static_cast<const uint16_t*>(a.kc);
  kp.vc = static_cast<const uint16_t*>(a.vc);
  kp.qf = a.q; kp.kbf = a.kb; kp.vbf = a.vb; kp.kcf = a.kc; kp.vcf = a.vc;
  kp.ctx_start = a.ctx_start; kp.ctx_len = a.ctx_len; kp.active = a.active;
  kp.shift = a.shift; kp.scale = a.scale;
  kp.qscale = kLog2e / sqrtf(static_cast<float>(a.d));
  kp.part_acc = ws;
  kp.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.part_acc_bytes);
  kp.causal = a.causal;
  kp.ctx_end = a.ctx_end; kp.kc_out = a.kc_out; kp.vc_out = a.vc_out;
  const int64_t units = static_cast<int64_t>(a.B) * a.Hkv * pl.row_blocks * pl.n_chunks;
  if (a.dtype == 0) {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(static_cast<unsigned>(units)), dim3(512), 0, st, kp);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(static_cast<unsigned>(units)), dim3(512), 0, st, kp);
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(static_cast<unsigned>(units)), dim3(64), 0, st, kp);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(static_cast<unsigned>(units)), dim3(64), 0, st, kp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MParams mp{};
  mp.B = a.B; mp.S = a.S; mp.Hq = a.Hq; mp.Hkv = a.Hkv; mp.G = G; mp.R = pl.rows; mp.D = a.d;
  mp.rows_per_unit = pl.rows_per_unit; mp.RB = pl.row_blocks; mp.NC = pl.n_chunks;
  mp.chunk = pl.chunk; mp.ctx_len = a.ctx_len; mp.active = a.active; mp.gate = a.gate;
  mp.residual = a.residual; mp.out = a.out; mp.lse = a.lse;
  mp.part_acc = kp.part_acc; mp.part_ml = kp.part_ml;
  const dim3 mg(static_cast<unsigned>(ceil_div(pl.rows_per_unit, a.d == 128 ? merge_rows_per_wg<128>()
                                                                         : merge_rows_per_wg<64>())),
                static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * pl.row_blocks));
  if (a.dtype == 0) {
    if (a.d == 128) hipLaunchKernelGGL((merge_kernel<uint16_t, 128>), mg, dim3(256), 0, st, mp);
    else hipLaunchKernelGGL((merge_kernel<uint16_t, 64>), mg, dim3(256), 0, st, mp);
  } else {
    if (a.d == 128) hipLaunchKernelGGL((merge_kernel<float, 128>), mg, dim3(256), 0, st, mp);
    else hipLaunchKernelGGL((merge_kernel<float, 64>), mg, dim3(256), 0, st, mp);
  }
  return hipGetLastError();
}

}  // namespace tt
