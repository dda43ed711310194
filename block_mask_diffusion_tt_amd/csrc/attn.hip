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
//     partials that the merge kernel combines in a fixed chunk order
//     (deterministic).
//
// bf16 kernel (gfx950 matrix cores, 64-wide waves): waves of 32 rows, 2, 4
// or 8 of them per workgroup (as many as the R rows of a KV head need, up to
// 256 rows; more rows make several row blocks), one workgroup per CU.
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
constexpr int kMaxWaves = 8;     // bf16 workgroups: up to 8 waves of 32 rows
constexpr int kRowsF32 = 64;     // rows per fp32 workgroup (1 wave, 1 row per lane)
constexpr int kMinChunk = 256;   // fewest context keys per unit (multiple of kTK): below
                                 // that, the fixed cost of a unit and of its partial dominate
constexpr int kModHeads = 16;    // largest query-head group whose adaLN vectors are staged in LDS
template <int D>
constexpr int kModStride = D + 4;   // floats per staged head (padded)
constexpr float kLog2e = 1.4426950408889634f;

struct KParams {
  int B, S, Hq, Hkv, G, R;
  int rows_per_unit, RB, NC, chunk, units;
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

// Logical unit of workgroup i (units are numbered (b, g, c, rb), row block
// fastest).  With several row blocks per group, workgroup i runs logical
// unit (i % 8) * ceil(U / 8) + i / 8: workgroups are dispatched to the 8 XCDs
// round-robin, so the row blocks of one context chunk start together on one
// XCD and read each K/V tile through its L2.  The grid then has 8 * ceil(U/8)
// workgroups and those past U have nothing to do.
__device__ __forceinline__ int unit_of_block(int i, int units, int RB) {
  if (RB == 1) return i;
  const int q = (units + 7) / 8;
  return (i % 8) * q + i / 8;
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
  un.rb = u % RB;
  int t = u / RB;
  un.c = t % NC;
  t /= NC;
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
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 16-byte global -> LDS copy through the direct path, from a wave-uniform
// base plus a per-lane byte offset (the SGPR-base form: no per-copy address
// arithmetic): lane i writes LDS bytes [lds + 16 i, lds + 16 i + 16).  Written
// in asm because the compiler would otherwise wait for every such copy in
// flight before any LDS read (it cannot tell the pipeline stages apart); the
// stage waits below are explicit.  The instruction has no register result.
// Marked non-temporal: the context K/V is read once per layer, so the caches
// need not keep it.  M0 is not in the clobber list: the compiler reserves it
// and warns that such a clobber is not honoured; instead the build fails if
// the compiler itself uses M0 anywhere in this file's kernels.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
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

// max / sum of a value over lanes l and l^32 (the two halves of a wave)
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keeps a value's computation before this point: an empty asm that reads and
// "writes" the register, so the compiler cannot sink the arithmetic that
// produces it into a later basic block.
#define TT_PIN(x) asm volatile("" : "+v"(x))

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. N-1.
template <int B, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < N) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, N>(f);
  }
}

// Slot order of the matrix products of a pipeline step (d/16 QK^T products
// kk and 2 * d/32 PV^T products j = ks * d/32 + dt, alternating, opening
// with two PV^T products): whether slot s is a QK^T product, and its kk or j.
template <int D>
struct SlotOrder;
template <>
struct SlotOrder<128> {
  static constexpr int N = 16;
  static constexpr int isq[16] = {0, 0, 1, 0, 1, 0, 1, 0, 1, 0, 1, 0, 1, 0, 1, 1};
  static constexpr int idx[16] = {0, 1, 0, 2, 1, 3, 2, 4, 3, 5, 4, 6, 5, 7, 6, 7};
};
template <>
struct SlotOrder<64> {
  static constexpr int N = 8;
  static constexpr int isq[8] = {0, 0, 1, 0, 1, 0, 1, 1};
  static constexpr int idx[8] = {0, 1, 0, 2, 1, 3, 2, 3};
};

template <int D, int NW>
struct Bf16Cfg {
  static constexpr int CH = D / 8;                 // 16-byte chunks per key row
  static constexpr int TILE = 64 * D * 2;          // bytes of one K (or V) tile of 64 keys
  static constexpr int NST = 4;                    // pipeline stages
  static constexpr int VREG = NST * TILE;          // V tiles follow the NST K tiles
  static constexpr int ROWS = 32 * NW;             // rows per workgroup (32 per wave)
  static constexpr int NT = 64 * NW;               // threads per workgroup
  static constexpr int CPT = 64 * CH / NT;         // copies per thread per tile tensor
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

// NW waves of 32 rows (NW = 8 for the 256 rows of S = 16 slots x 16 heads;
// fewer for smaller blocks, so that no wave multiplies rows that do not exist).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_bf16_kernel(KParams p) {
  using C = Bf16Cfg<D, NW>;
  constexpr int KSTEPS = D / 16;   // MFMA k-steps of QK^T
  constexpr int DT = D / 32;       // 32-channel tiles of the output
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::SMEM];
  __shared__ __attribute__((aligned(16))) float smod[2 * kModHeads * kModStride<D>];

  const int ul = unit_of_block(blockIdx.x, p.units, p.RB);
  if (ul >= p.units) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const int64_t kstride = static_cast<int64_t>(p.Hkv) * D;
  TT_LDS uint8_t* const lsm = (TT_LDS uint8_t*)(smem);  // address-space cast
  // this lane's row: rl within the unit's row block, row within the group
  const int rl = wave * 32 + l32;
  const int row = (ul % p.RB) * C::ROWS + rl;

  // Q' = (q * (1 + scale) + shift) * log2(e)/sqrt(d), rounded to bf16;
  // lane l32 holds its row.  The query and modulation loads depend on the
  // unit's sequence, head and row block only (its number), so they go out
  // first, before the lengths decide whether the unit has work.  Rows past R
  // read row 0 and are zeroed.
  //   The modulation vectors depend on the head only, so every wave would
  // load the same G heads: with G <= kModHeads the workgroup stages the
  // unit's G x d scale and shift in LDS once (contiguous in memory, one
  // 16-byte load per thread and vector at the headline shape; rows padded by
  // 16 bytes to spread the heads over the banks) and every lane reads its
  // head from there after the barrier that makes tiles 0 and 1 visible.
  // Larger groups load per lane (each lane its row's head).
  constexpr int MPER = (kModHeads * D / 4 + C::NT - 1) / C::NT;
  const bool has_sc = p.scale != nullptr, has_sh = p.shift != nullptr;
  const bool has_mod = has_sc || has_sh;
  const bool staged = has_mod && p.G <= kModHeads;
  const bool valid = row < p.R;
  uint4 qraw[KSTEPS];
  float4 sca[KSTEPS][2], sha[KSTEPS][2];
  float4 msc[MPER], msh[MPER];
  {
    const int t = ul / p.RB / p.NC;
    const int ug = t % p.Hkv, ub = t / p.Hkv;
    const int h = ug * p.G + (valid ? row % p.G : 0);
    const int s = valid ? row / p.G : 0;
    const uint16_t* qrow = p.q + ((static_cast<int64_t>(ub) * p.S + s) * p.Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qraw[kk] = *reinterpret_cast<const uint4*>(qrow + kk * 16 + half * 8);
    // a missing vector reads the present one (ignored below), so that one
    // branch holds every modulation load
    const float* scv = has_sc ? p.scale : p.shift;
    const float* shv = has_sh ? p.shift : p.scale;
    if (staged) {
      const int n4 = p.G * D / 4;
      const int64_t base = (static_cast<int64_t>(ub) * p.Hq + ug * p.G) * D;
#pragma unroll
      for (int i = 0; i < MPER; ++i) {
        const int e = tid + i * C::NT;
        msc[i] = e < n4 ? *reinterpret_cast<const float4*>(scv + base + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
        msh[i] = e < n4 ? *reinterpret_cast<const float4*>(shv + base + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else if (has_mod) {
      const int64_t ada = (static_cast<int64_t>(ub) * p.Hq + h) * D + half * 8;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          sca[kk][i] = *reinterpret_cast<const float4*>(scv + ada + kk * 16 + 4 * i);
          sha[kk][i] = *reinterpret_cast<const float4*>(shv + ada + kk * 16 + 4 * i);
        }
    }
  }
  Unit un;
  if (!decode_unit(ul, p.Hkv, p.RB, p.NC, p.chunk, p.ctx_len, p.active, un)) return;
  append_block_kv(p, un, D, 2);
  // block keys visible to this lane's row: all S, or slots 0..s when causal
  // (rows past R take all S, so every row has a finite maximum)
  const int blk_valid = (p.causal && row < p.R) ? row / p.G + 1 : p.S;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lsm));

  // ---- tiles: the block's S keys first (chunk 0), then 64-key context tiles
  const int n_ctx_tiles = (un.k_end - un.k_beg + kTK - 1) / kTK;
  const int n_tiles = (un.has_blk ? 1 : 0) + n_ctx_tiles;
  const int nh = 2 * n_tiles;   // 32-key halves
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

  // Scores are kept relative to each row's running reference mu: the QK^T
  // accumulation starts from -mu (negmu, all 16 entries of a lane belong to
  // one row), so no subtraction is needed before the exponentials.
  f32x16 acc[DT];
  float mu = 0.f, lsum = 0.f;
  f32x16 negmu;
#pragma unroll
  for (int r = 0; r < 16; ++r) negmu[r] = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  // Half g (32 keys) of the unit is half g & 1 of tile g >> 1, in stage
  // (g >> 1) % NST.  K operand kk of half g (A of S^T = K Q'^T):
  auto kread = [&](int g, int kk) {
    TT_LDS const uint8_t* a = lsm + ((g >> 1) % C::NST) * C::TILE + (g & 1) * 32 * C::CH * 16 + kbase + kk * 2 * 16 * 16;
    return *reinterpret_cast<TT_LDS const bf16x8*>(a);
  };
  // V^T operand (A of O^T += V^T P^T) of 16-key step ks, channel tile dt of
  // half g: two transpose reads
  auto vread = [&](int g, int ks, int dt) {
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    TT_LDS uint8_t* a = lsm + ((g >> 1) % C::NST) * C::TILE + (g & 1) * 8 * 4 * C::CH * 16 + vbase +
                        ks * 4 * 4 * C::CH * 16 + dt * 4 * 4 * 16;
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<TT_LDS v4i16*>(a));
    const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<TT_LDS v4i16*>(a + 2 * 4 * C::CH * 16));
    const v8i16 w8 = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
    return __builtin_bit_cast(bf16x8, w8);
  };
  // keys at or past the valid count of the tile holding half g are masked to
  // -inf (key of accumulator r in half g&1 is (g&1)*32 + 4*half + 8*(r/4) + r%4)
  auto mask_half = [&](f32x16& sc, int g) {
    const int nvalid = tile_valid(g >> 1);
    const int lim = nvalid - (g & 1) * 32 - 4 * half;
    if (lim < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
    }
  };
  // P = 2^S (scores relative to mu), rounded to bf16: the B operand of P^T
  auto pack = [&](const f32x16& e, int r0) {
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 pr = {static_cast<__bf16>(e[r0 + 2 * i]), static_cast<__bf16>(e[r0 + 2 * i + 1])};
      pk[i] = __builtin_bit_cast(uint32_t, pr);
    }
    return __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
  };
  auto row_sum = [&](const f32x16& e) {
    float s0 = e[0], s1 = e[1];
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      s0 += e[r];
      s1 += e[r + 1];
    }
    return s0 + s1;
  };
  constexpr int LD = 2 * C::CPT;  // copies per thread per tile

  // Software pipeline over halves (per wave).  Step h runs one stream of
  // matrix products that interleaves the PV^T products of half h (DT channel
  // tiles x 2 k-steps, independent) with the dependent QK^T chain of half
  // h+2 (D/16 products), while the vector unit turns the scores of half h+1
  // into P(h+1)
  // (exponentials, packs, the row sum): no product waits for the softmax and
  // no exponential for a product.  The stream opens with two PV^T products,
  // which gives the previous step's last QK^T products time to land before
  // the exponentials need their scores.  Every operand is read from LDS two
  // product slots before its use.
  //   The running reference mu is raised only when a half's row sum
  // exceeds 2^8 (some probability above 2^8, or many large ones): that rare
  // step recomputes S(h+1) relative to the old mu, raises mu to the row
  // maximum, rescales the accumulator and the sum, and shifts S(h+2).
  //   Tiles stream HBM -> LDS in a 4-stage ring.  At the start of tile t
  // (step 2t) the workgroup waits until tile t+1 is visible (the K operands
  // of steps 2t and 2t+1) and refills the stage of tile t-1, whose last
  // reads were in step 2t-1, with tile t+3: two tiles are in flight while
  // two are read.
  bf16x8 kop[KSTEPS];      // K operands of the QK^T chain in flight
  bf16x8 vop[2 * DT];      // V^T operands of the PV^T products, j = ks * DT + dt
  f32x16 scr[2];           // scores of halves of even / odd index
  bf16x8 pb[2][2];         // P of halves of even / odd index (two k-steps)
  bf16x8 qf[KSTEPS];
  for (int t = 0; t < (n_tiles < 2 ? n_tiles : 2); ++t) issue(t);
  if (staged) {
    // (the wait for these values also covers the copies just issued)
#pragma unroll
    for (int i = 0; i < MPER; ++i) {
      const int e = tid + i * C::NT;
      if (e < p.G * D / 4) {
        const int j = (4 * e) / D, c = (4 * e) % D;
        *reinterpret_cast<float4*>(&smod[j * kModStride<D> + c]) = msc[i];
        *reinterpret_cast<float4*>(&smod[(kModHeads + j) * kModStride<D> + c]) = msh[i];
      }
    }
  }
  // tiles 0 and 1 (and the staged vectors) visible, then tiles 2 and 3 start
  wait_vmem<0>();
  __syncthreads();
  for (int t = 2; t < (n_tiles < C::NST ? n_tiles : C::NST); ++t) issue(t);
  if (staged) {
    const int j = valid ? row % p.G : 0;
    const float* scl = &smod[j * kModStride<D> + half * 8];
    const float* shl = &smod[(kModHeads + j) * kModStride<D> + half * 8];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        sca[kk][i] = *reinterpret_cast<const float4*>(scl + kk * 16 + 4 * i);
        sha[kk][i] = *reinterpret_cast<const float4*>(shl + kk * 16 + 4 * i);
      }
  }
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const uint4 w = qraw[kk];
    float v[8] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u),
                  __uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
                  __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u)};
    if (has_mod) {
      const float4 a0 = sca[kk][0], a1 = sca[kk][1];
      const float4 b0 = sha[kk][0], b1 = sha[kk][1];
      const float sc8[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float sh8[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (has_sc) v[i] *= 1.f + sc8[i];
        if (has_sh) v[i] += sh8[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[kk][i] = static_cast<__bf16>(valid ? v[i] * p.qscale : 0.f);
  }
  // prologue: S(0), S(1); the reference mu is S(0)'s row maximum (finite:
  // the first half of a unit's first tile always holds a valid key)
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) kop[kk] = kread(0, kk);
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    scr[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[kk], kk == 0 ? negmu : scr[0], 0, 0, 0);
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) kop[kk] = kread(1, kk);
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    scr[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[kk], kk == 0 ? negmu : scr[1], 0, 0, 0);
  vop[0] = vread(0, 0, 0);
  vop[1] = vread(0, 0, 1);
  mask_half(scr[0], 0);
  {
    float m = fmaxf(scr[0][0], scr[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m = fmaxf(m, fmaxf(scr[0][r], scr[0][r + 1]));
    mu = xhalf_max(m);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    scr[0][r] = __builtin_amdgcn_exp2f(scr[0][r] - mu);
    scr[1][r] -= mu;
    negmu[r] = -mu;
  }
  pb[0][0] = pack(scr[0], 0);
  pb[0][1] = pack(scr[0], 8);
  lsum = row_sum(scr[0]);

  // The rare step: S(g) = scores of half g relative to the old mu,
  // recomputed from LDS (sn already holds its exponentials); mu is raised to
  // the row maximum where that is positive, and S(g+1) (s2) shifted along.
  auto raise_mu = [&](int g, f32x16& sn, f32x16& s2, bf16x8 (&pn)[2], float& esum) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const bf16x8 k1 = kread(g, kk);
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[kk], kk == 0 ? negmu : sn, 0, 0, 0);
    }
    mask_half(sn, g);
    float m = fmaxf(sn[0], sn[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m = fmaxf(m, fmaxf(sn[r], sn[r + 1]));
    const float up = fmaxf(xhalf_max(m), 0.f);
    const float alpha = __builtin_amdgcn_exp2f(-up);
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    mu += up;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sn[r] = __builtin_amdgcn_exp2f(sn[r] - up);
      s2[r] -= up;
      negmu[r] = -mu;
    }
    pn[0] = pack(sn, 0);
    pn[1] = pack(sn, 8);
    esum = row_sum(sn);
  };

  // Step h (E = h & 1).  EDGE: half h+1 may be partial (first or last tile)
  // or missing, half h+2 may be missing (its products then run on stale LDS
  // data and are never used).
  auto step = [&](int h, auto odd_c, auto edge_c) {
    constexpr int E = decltype(odd_c)::value;
    constexpr bool EDGE = decltype(edge_c)::value;
    f32x16& sn = scr[E ^ 1];       // S(h+1) -> exponentials
    f32x16& s2 = scr[E];           // S(h+2) (the stale S(h) dies here)
    bf16x8 (&pc)[2] = pb[E];       // P(h)
    bf16x8 (&pn)[2] = pb[E ^ 1];
    const int t = h >> 1;
    if (!E && t > 0) {
      if (t + 2 < n_tiles) wait_vmem<LD>();
      else wait_vmem<0>();
      __syncthreads();
      if (t + C::NST - 1 < n_tiles) issue(t + C::NST - 1);
    }
    if (EDGE) mask_half(sn, h + 1);
    // vector work: the 16 exponentials spread over the slots (from slot 1;
    // the previous step's last QK^T products land meanwhile), each one's
    // row-sum term two slots later, the packs once the values exist
    using SO = SlotOrder<D>;
    constexpr int NS = SO::N;
    constexpr int EPS = 16 / NS;      // exponentials per slot
    float rs0, rs1;                   // the row sum of P(h+1), two chains
    static_for<0, NS>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      constexpr int x = SO::idx[s];
      if constexpr (SO::isq[s] != 0)
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[x], qf[x], x == 0 ? negmu : s2, 0, 0, 0);
      else
        acc[x % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[x], pc[x / DT], acc[x % DT], 0, 0, 0);
      // the operand of the product two slots ahead (the next step's first
      // two PV^T products for the last two slots)
      if constexpr (s + 2 < NS) {
        constexpr int y = SO::idx[s + 2];
        if constexpr (SO::isq[s + 2] != 0) kop[y] = kread(h + 2, y);
        else vop[y] = vread(h, y / DT, y % DT);
      } else {
        constexpr int y = SO::idx[s + 2 - NS];
        vop[y] = vread(h + 1, y / DT, y % DT);
      }
      // exponentials e0 .. e1-1 in this slot (none in slot 0, the rest in
      // the last one); the row-sum terms of those of two slots back
      constexpr int e0 = s == 0 ? 0 : (s - 1) * EPS;
      constexpr int e1 = s == 0 ? 0 : (s == NS - 1 ? 16 : s * EPS);
      constexpr int a0 = s < 3 ? 0 : (s - 3) * EPS;
      constexpr int a1 = s < 3 ? 0 : (s - 2) * EPS;
      static_for<e0, e1>([&](auto r_c) {
        constexpr int r = decltype(r_c)::value;
        sn[r] = __builtin_amdgcn_exp2f(sn[r]);
      });
      static_for<a0, a1>([&](auto r_c) {
        constexpr int r = decltype(r_c)::value;
        if constexpr (r == 0) rs0 = sn[0];
        else if constexpr (r == 1) rs1 = sn[1];
        else if constexpr (r & 1) rs1 += sn[r];
        else rs0 += sn[r];
      });
      if constexpr (s == 8 / EPS + 1) {   // e0..e7 exist
        pn[0] = pack(sn, 0);
        // kept here: the rare branch below redefines pn, and the compiler
        // would otherwise sink the packs to the next step's first products
        TT_PIN(pn[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<(NS - 3) * EPS, 16>([&](auto r_c) {
      constexpr int r = decltype(r_c)::value;
      if constexpr (r & 1) rs1 += sn[r];
      else rs0 += sn[r];
    });
    pn[1] = pack(sn, 8);
    TT_PIN(pn[1]);
    float esum = rs0 + rs1;
    if (!EDGE || h + 1 < nh) {
      if (__builtin_expect(__any(esum > 256.f), 0)) raise_mu(h + 1, sn, s2, pn, esum);
      lsum += esum;
    }
  };
  // tile 0 and the last two tiles take the edge steps, the rest the
  // steady-state ones (three loops, so each has one body)
  step(0, std::integral_constant<int, 0>{}, std::true_type{});
  step(1, std::integral_constant<int, 1>{}, std::true_type{});
  int t = 1;
  for (; t + 2 < n_tiles; ++t) {
    step(2 * t, std::integral_constant<int, 0>{}, std::false_type{});
    step(2 * t + 1, std::integral_constant<int, 1>{}, std::false_type{});
  }
  for (; t < n_tiles; ++t) {
    step(2 * t, std::integral_constant<int, 0>{}, std::true_type{});
    step(2 * t + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }

  // ---- partials: (max, sum) per row and the unnormalised accumulator, in
  // the unit's slot ((b * Hkv + g) * RB + rb) * NC + c.  Lanes of rows past R
  // compute along (their values are finite) but store nothing.
  const float ltot = xhalf_sum(lsum);
  const bool live = row < p.R;
  const int64_t u = ((static_cast<int64_t>(un.b) * p.Hkv + un.g) * p.RB + un.rb) * p.NC + un.c;
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
  if (live && half == 0)
    *reinterpret_cast<float4*>(p.part_ml + (u * C::ROWS + rl) * 4) =
        make_float4(mu, ltot, static_cast<float>(k), 0.f);
  // The fp16 rows go out through LDS: each wave writes its 32 rows x d into
  // a private half of a K or V tile region of a stage that no wave reads or
  // copies into any more (the stages of the three tiles before the last: no
  // copy is pending after the last tiles' waits, and after the barrier at the
  // last tile's start every wave reads that tile only; a unit with fewer
  // tiles never filled them), then stores whole 16-byte row chunks, 1 KB per
  // instruction, instead of 8-byte pieces scattered over 32 rows.  The
  // 16-byte chunk index is XOR-swizzled with the row to spread the rows over
  // the LDS banks.
  {
    constexpr int RB16 = D / 8;            // 16-byte chunks per row
    const int tl = n_tiles - 1;
    const int piece = wave >> 1;           // K, V of stage tl+1, then K, V of stage tl+2
    const int stage = (tl + 1 + (piece >> 1)) % C::NST;
    TT_LDS uint8_t* const wb = lsm + (piece & 1) * C::VREG + stage * C::TILE + (wave & 1) * (C::TILE / 2);
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half4 hv = {static_cast<_Float16>(acc[dt][4 * j] * sc), static_cast<_Float16>(acc[dt][4 * j + 1] * sc),
                          static_cast<_Float16>(acc[dt][4 * j + 2] * sc), static_cast<_Float16>(acc[dt][4 * j + 3] * sc)};
        const int c = dt * 4 + j;
        *reinterpret_cast<TT_LDS u32x2*>(wb + l32 * (D * 2) + ((c ^ (l32 & (RB16 - 1))) * 16) + half * 8) =
            __builtin_bit_cast(u32x2, hv);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint16_t* const dst = static_cast<uint16_t*>(p.part_acc) + (u * C::ROWS + wave * 32) * D;
#pragma unroll
    for (int i = 0; i < 32 * RB16 / 64; ++i) {
      const int idx = i * 64 + lane;
      const int r = idx / RB16, c = idx % RB16;
      const u32x4 v = *reinterpret_cast<const TT_LDS u32x4*>(wb + r * (D * 2) + ((c ^ (r & (RB16 - 1))) * 16));
      if (un.rb * C::ROWS + wave * 32 + r < p.R)
        *reinterpret_cast<u32x4*>(dst + r * D + c * 8) = v;
    }
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
  const int ul = unit_of_block(blockIdx.x, p.units, p.RB);
  if (ul >= p.units || !decode_unit(ul, p.Hkv, p.RB, p.NC, p.chunk, p.ctx_len, p.active, un)) return;
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
  const int64_t u = ((static_cast<int64_t>(un.b) * p.Hkv + un.g) * p.RB + un.rb) * p.NC + un.c;
  *reinterpret_cast<float4*>(p.part_ml + (u * kRowsF32 + tid) * 4) = make_float4(m, l, 0.f, 0.f);
  float* dst = static_cast<float*>(p.part_acc) + (u * kRowsF32 + tid) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int dd = 0; dd < D; ++dd) dst[dd] = acc[dd] * inv;
}

// ------------------------------------------------------------------ merge
// o = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, combined in chunk
// order; lse = ln2 * (M + log2 sum); out = residual + gate * o.
// 8 consecutive output-type values as one 16-byte access for bf16 (two for
// fp32): each 16-byte piece of an output row is written by one instruction,
// so the lines a wave writes arrive whole (two 8-byte stores per piece made
// the memory side fetch the output's lines before writing them).
template <typename OutT>
__device__ __forceinline__ void load8(const OutT* src, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* src, float (&v)[8]) {
  const float4 x = reinterpret_cast<const float4*>(src)[0], y = reinterpret_cast<const float4*>(src)[1];
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* src, float (&v)[8]) {
  const uint4 x = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename OutT>
__device__ __forceinline__ void store8(OutT* dst, const float (&v)[8]);

template <>
__device__ __forceinline__ void store8<float>(float* dst, const float (&v)[8]) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* dst, const float (&v)[8]) {
  typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
  bf16x8v b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = static_cast<__bf16>(v[i]);
  *reinterpret_cast<uint4*>(dst) = __builtin_bit_cast(uint4, b);
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
template <typename T>
struct TypeTag { using type = T; };
template <int D>
constexpr int merge_rows_per_wg() { return 256 / (D / (4 * kMergeQuads)); }

// NB: chunk partials loaded together (2, 4, 8 or 16: the smallest that
// covers the plan's chunks, 16 beyond).
//   kMany (NB = 16, plans of more than 8 chunks: few rows, many partials per
// row, a latency-bound merge): the gate and residual loads go out before the
// chunks are combined, and the chunk loads carry no branches (chunks past n
// read chunk n - 1 again and are dropped by selection; a missing gate or
// residual reads a valid stand-in that is ignored), so the merge waits
// for memory once instead of three times (one sequence of 4096 tokens, 16
// chunks per KV head: 8.7 -> 5.6 us).  With few chunks the merge is
// bandwidth-bound and keeps its loads as they are (the same change there
// cost 0.5 us at 64 x 8192 tokens).
template <typename OutT, int D, int NB>
__global__ __launch_bounds__(256) void merge_kernel(MParams p) {
  constexpr int CPT = 4 * kMergeQuads;   // channels per thread
  constexpr int Q = kMergeQuads;         // 16-byte loads per thread per chunk
  constexpr int TPR = D / CPT;           // threads per row
  constexpr bool kMany = NB >= 16;
  static_assert(CPT == 8, "the epilogue moves 8 channels per thread");
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
  float gv[CPT], rv[CPT];
  if constexpr (kMany) {
    const int s = row / p.G, h = g * p.G + row % p.G;
    const int64_t orow = (static_cast<int64_t>(b) * p.S + s) * p.Hq + h;
    const float* const gp = p.gate ? p.gate + (static_cast<int64_t>(b) * p.Hq + h) * D + c0 : p.part_ml;
    // stand-ins: the records' first floats, and this row's chunk-0 partial
    // (same element width as OutT, loaded by this thread anyway)
    const OutT* const rp = p.residual ? static_cast<const OutT*>(p.residual) + orow * D + c0
                                      : static_cast<const OutT*>(p.part_acc) + (u0 * p.rows_per_unit + rl) * D + c0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(gp + 4 * q);
      gv[4 * q] = x.x; gv[4 * q + 1] = x.y; gv[4 * q + 2] = x.z; gv[4 * q + 3] = x.w;
    }
    load8<OutT>(rp, rv);
  }
  // chunk c contributes 2^(m_c - M) l_c o_c, M the largest m_c; its stored
  // partial is o_c 2^-k_c (fp16 for bf16 output, fp32 for fp32 output).
  // One pass over the chunks, NB at a time (all their loads issued
  // together), the running sums rescaled when a batch raises the maximum.
  float M = -INFINITY, L = 0.f;
  float o[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) o[i] = 0.f;
  for (int cb = 0; cb < n; cb += NB) {
    float4 ml[NB];
    float a[NB][CPT];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (kMany) {
        const int64_t base = (u0 + min(cb + j, n - 1)) * p.rows_per_unit + rl;
        ml[j] = *reinterpret_cast<const float4*>(p.part_ml + base * 4);
        load_part<OutT, CPT>(p.part_acc, base * D + c0, a[j]);
      } else if (cb + j < n) {
        const int64_t base = (u0 + cb + j) * p.rows_per_unit + rl;
        ml[j] = *reinterpret_cast<const float4*>(p.part_ml + base * 4);
        load_part<OutT, CPT>(p.part_acc, base * D + c0, a[j]);
      } else {
        ml[j] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < CPT; ++i) a[j][i] = 0.f;
      }
    }
    if constexpr (kMany) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const bool in = cb + j < n;
        ml[j].x = in ? ml[j].x : -INFINITY;
        ml[j].y = in ? ml[j].y : 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) a[j][i] = in ? a[j][i] : 0.f;
      }
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < NB; ++j) Mb = fmaxf(Mb, ml[j].x);
    const float r = exp2f(M - Mb);   // 0 on the first batch (M = -inf)
    L *= r;
#pragma unroll
    for (int i = 0; i < CPT; ++i) o[i] *= r;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float wl = exp2f(ml[j].x - Mb) * ml[j].y;
      L += wl;
      const float coef = ldexpf(wl, static_cast<int>(ml[j].z));
#pragma unroll
      for (int i = 0; i < CPT; ++i) o[i] = fmaf(coef, a[j][i], o[i]);
    }
    M = Mb;
  }
  const float inv = 1.f / L;
  const int s = row / p.G, h = g * p.G + row % p.G;
  const int64_t orow = (static_cast<int64_t>(b) * p.S + s) * p.Hq + h;
  const float* gp = p.gate ? p.gate + (static_cast<int64_t>(b) * p.Hq + h) * D + c0 : nullptr;
  const OutT* rp = p.residual ? static_cast<const OutT*>(p.residual) + orow * D + c0 : nullptr;
  OutT* op = static_cast<OutT*>(p.out) + orow * D + c0;
  float v[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) v[i] = o[i] * inv;
  if (gp) {
    if constexpr (!kMany) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 x = *reinterpret_cast<const float4*>(gp + 4 * q);
        gv[4 * q] = x.x; gv[4 * q + 1] = x.y; gv[4 * q + 2] = x.z; gv[4 * q + 3] = x.w;
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) v[i] *= gv[i];
  }
  if (rp) {
    if constexpr (!kMany) load8<OutT>(rp, rv);
#pragma unroll
    for (int i = 0; i < CPT; ++i) v[i] += rv[i];
  }
  store8<OutT>(op, v);
  if (p.lse && c0 == 0) p.lse[orow] = 0.6931471805599453f * (M + log2f(L));
}

}  // namespace

AttnPlan attn_plan(int B, int S, int Hq, int Hkv, int d, int dtype, int max_ctx_len) {
  AttnPlan pl{};
  const int G = Hq / Hkv;
  pl.rows = S * G;
  // bf16: waves of 32 rows, as few as the rows need (a power of two from 2
  // to kMaxWaves); fp32: one wave of 64 rows
  int nw = 2;
  while (nw < kMaxWaves && 32 * nw < pl.rows) nw *= 2;
  pl.rows_per_unit = dtype == 0 ? 32 * nw : kRowsF32;
  pl.row_blocks = static_cast<int>(ceil_div(pl.rows, pl.rows_per_unit));
  const int64_t groups = static_cast<int64_t>(B) * Hkv * pl.row_blocks;
  const int64_t want = ceil_div(device_cus(), groups);
  int64_t chunk = max_ctx_len > 0 ? ceil_div(max_ctx_len, want < 1 ? 1 : want) : kTK;
  chunk = static_cast<int64_t>(align_up(static_cast<size_t>(chunk), kTK));
  if (chunk < kMinChunk) chunk = kMinChunk;
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
  kp.units = static_cast<int>(units);
  // several row blocks per group: the grid is padded to a multiple of 8 for
  // the XCD-aware unit order (unit_of_block)
  const unsigned grid = static_cast<unsigned>(pl.row_blocks > 1 ? 8 * ceil_div(units, 8) : units);
  if (a.dtype == 0) {
    const int nw = pl.rows_per_unit / 32;
    if (a.d == 128) {
      if (nw == 8) hipLaunchKernelGGL((attn_bf16_kernel<128, 8>), dim3(grid), dim3(512), 0, st, kp);
      else if (nw == 4) hipLaunchKernelGGL((attn_bf16_kernel<128, 4>), dim3(grid), dim3(256), 0, st, kp);
      else hipLaunchKernelGGL((attn_bf16_kernel<128, 2>), dim3(grid), dim3(128), 0, st, kp);
    } else {
      if (nw == 8) hipLaunchKernelGGL((attn_bf16_kernel<64, 8>), dim3(grid), dim3(512), 0, st, kp);
      else if (nw == 4) hipLaunchKernelGGL((attn_bf16_kernel<64, 4>), dim3(grid), dim3(256), 0, st, kp);
      else hipLaunchKernelGGL((attn_bf16_kernel<64, 2>), dim3(grid), dim3(128), 0, st, kp);
    }
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(64), 0, st, kp);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(64), 0, st, kp);
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
  const int nb = pl.n_chunks <= 2 ? 2 : pl.n_chunks <= 4 ? 4 : pl.n_chunks <= 8 ? 8 : 16;
  auto merge = [&](auto out_c, auto d_c, auto nb_c) {
    using OutT = typename decltype(out_c)::type;
    hipLaunchKernelGGL((merge_kernel<OutT, decltype(d_c)::value, decltype(nb_c)::value>), mg,
                       dim3(256), 0, st, mp);
  };
  auto by_nb = [&](auto out_c, auto d_c) {
    if (nb == 2) merge(out_c, d_c, std::integral_constant<int, 2>{});
    else if (nb == 4) merge(out_c, d_c, std::integral_constant<int, 4>{});
    else if (nb == 8) merge(out_c, d_c, std::integral_constant<int, 8>{});
    else merge(out_c, d_c, std::integral_constant<int, 16>{});
  };
  auto by_d = [&](auto out_c) {
    if (a.d == 128) by_nb(out_c, std::integral_constant<int, 128>{});
    else by_nb(out_c, std::integral_constant<int, 64>{});
  };
  if (a.dtype == 0) by_d(TypeTag<uint16_t>{});
  else by_d(TypeTag<float>{});
  return hipGetLastError();
}

}  // namespace tt
