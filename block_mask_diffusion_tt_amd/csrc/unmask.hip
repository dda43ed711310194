// Confidence unmasking over the vocabulary: one HBM pass per masked row
// (max, lowest-index argmax, sum of exp((l - max)/tau)), then a per-sequence
// commit / re-mask decision that is exact with respect to fp64.
//
// [keyframe] key point 3: all masked slots of a block are predicted at once,
// confident tokens are committed step by step, the undetermined rest is
// masked again.  [dothoosh] benchmark paragraph: the threshold gamma sets how
// many tokens a step commits.  [news] code example: confidence_threshold=0.8,
// temperature=0.1, mask_token_id=3.
//
// Kernels
//   rowreduce  grid (splits, B*S), 256 threads.  Each workgroup scans one
//              fixed slice of one masked row with 16-byte loads; every thread
//              keeps (max, first index of max, sum of exp2((x - max) * c))
//              with c = log2(e)/tau, rescaling its sum when its max grows.
//              Per-thread partials combine in a fixed tree (deterministic).
//   decide     grid B, 256 threads.  Combines the slices of each row in
//              slice order, p = 1/Z in fp32, then recomputes in fp64 every
//              row whose p lies within kDelta of gamma -- and, when no row
//              passes and a second row lies within 2*kDelta of the best p,
//              every row in that band -- so the commit set is the one fp64
//              arithmetic gives.  kDelta = 2^-14
//              is about ten times the worst-case fp32 error of p at
//              V = 131072: the longest chain of roundings into Z is about 80
//              additions (64 group sums per thread at one split, the 3-level
//              group tree, the 8-level thread/wave tree, the slice merge),
//              at most 80 * 2^-24 relative, plus the exp2 argument rounding
//              (|x - m| * c * 2^-24, under 2e-6 for the terms that matter)
//              and one rounding of 1/Z: about 6e-6 in all.
//
// Temperature sampling (the same decision rule, a different prediction):
//   rowsample  grid (splits, B*S) as rowreduce, 256 threads.  Each
//              workgroup streams its slice in passes of 8192 tokens (32 per
//              thread, held in registers, the next pass's loads in flight):
//              the pass maximum first (one barrier), so Z and the Gumbel-max
//              candidates -- the only tokens that can win, those within
//              tau * (Gumbel range) of the running maximum -- are known
//              against it.  Only candidates draw their Philox4x32-10 noise
//              (a few per row), so the pass stays one read of the row.
//   decide     the same kernel as above with the slices' (max, Z, best
//              perturbed score, second best, token, logit); rows whose best
//              two perturbed scores lie within kKeyBand * (1 + |max| +
//              20 tau) get their candidates rescored in fp64 first.
#include <float.h>
#include <limits.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kThreads = 256;
constexpr float kDelta = 6.103515625e-05f;  // 2^-14
// Band of the perturbed scores l + tau G within which the sampled token is
// settled in fp64: kKeyBand (1 + |max| + 20 tau).  An fp32 score is off by at
// most about 2^-23 (|l| + 17 tau) + 2^-20 tau (two rounded logarithms, one
// product, one sum), 60 times less than the band.
constexpr float kKeyBand = 7.62939453125e-06f;  // 2^-17

struct RowPart {
  float m;   // max of the slice
  float z;   // sum of exp2((x - m) * c) over the slice
  int arg;   // lowest index attaining m (INT_MAX if the slice is empty)
  int pad;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void merge(float& m, float& z, int& a, float m2, float z2, int a2,
                                      float c) {
  const float M = fmaxf(m, m2);
  const float zz = z * fast_exp2((m - M) * c) + z2 * fast_exp2((m2 - M) * c);
  a = (m > m2) ? a : ((m2 > m) ? a2 : min(a, a2));
  m = M;
  z = zz;
}

// Eight consecutive logits starting at element i (16-byte aligned in the vector path).
template <typename T>
__device__ __forceinline__ void load8(const T* x, int64_t i, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* x, int64_t i, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(x + i);
  v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
  v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xffff0000u);
  v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xffff0000u);
}

template <>
__device__ __forceinline__ void load8<float>(const float* x, int64_t i, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(x + i);
  const float4 b = *reinterpret_cast<const float4*>(x + i + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Eight consecutive logits as loaded (raw words), unpacked to fp32 when used,
// so a load can stay in flight while earlier data is processed.
template <typename T>
struct Raw8;

template <>
struct Raw8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* x, int64_t i) {
    w = *reinterpret_cast<const uint4*>(x + i);
  }
  __device__ __forceinline__ void unpack(float (&v)[8]) const {
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
    v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xffff0000u);
    v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};

template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* x, int64_t i) {
    a = *reinterpret_cast<const float4*>(x + i);
    b = *reinterpret_cast<const float4*>(x + i + 4);
  }
  __device__ __forceinline__ void unpack(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

__device__ __forceinline__ float load1(const uint16_t* x, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(x[i]) << 16);
}
__device__ __forceinline__ float load1(const float* x, int64_t i) { return x[i]; }

template <typename T>
__global__ __launch_bounds__(kThreads) void rowreduce_kernel(
    const T* __restrict__ logits, int64_t row_stride, int V, const uint8_t* __restrict__ masked,
    float c, int split_len, int splits, int vec_ok, RowPart* __restrict__ part) {
  const int row = blockIdx.y;
  if (!masked[row]) return;
  const int split = blockIdx.x;
  const int beg = split * split_len;
  const int end = min(V, beg + split_len);
  const T* x = logits + static_cast<int64_t>(row) * row_stride;
  float m = -FLT_MAX, z = 0.f;
  int a = INT_MAX;
  int scalar_from = beg;
  // one group of 8 consecutive logits, in increasing index order
  auto group = [&](const float (&v)[8], int base) {
    const float m8 = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                           fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
    if (m8 > m) {
      z *= fast_exp2((m - m8) * c);
      m = m8;
      int j = 7;
#pragma unroll
      for (int k = 6; k >= 0; --k) j = (v[k] == m8) ? k : j;
      a = base + j;
    }
    float e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = fast_exp2((v[k] - m) * c);
    z += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  };
  if (vec_ok) {
    const int ngroups = (end - beg) >> 3;
    int gi = threadIdx.x;
    // uniform trips of four groups per thread (each lane still takes its
    // groups tid, tid + 256, ... in index order, the remainder in the loop
    // below); the next trip's loads are issued before this trip's arithmetic,
    // into the other of two raw buffers (a copy between buffers would wait for
    // its loads).  The last trip's fetch repeats its own addresses (in bounds,
    // unused).
    const int trips = ngroups / (4 * kThreads);
    auto fetch = [&](Raw8<T> (&r)[4], int g) {
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u].load(x, beg + ((g + u * kThreads) << 3));
    };
    auto trip = [&](const Raw8<T> (&r)[4], int g) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float v[8];
        r[u].unpack(v);
        group(v, beg + ((g + u * kThreads) << 3));
      }
    };
    if (trips > 0) {
      Raw8<T> ra[4], rb[4];
      fetch(ra, gi);
      for (int t = 0;;) {
        fetch(rb, t + 1 < trips ? gi + 4 * kThreads : gi);
        trip(ra, gi);
        gi += 4 * kThreads;
        if (++t == trips) break;
        fetch(ra, t + 1 < trips ? gi + 4 * kThreads : gi);
        trip(rb, gi);
        gi += 4 * kThreads;
        if (++t == trips) break;
      }
    }
    for (; gi < ngroups; gi += kThreads) {
      float v[8];
      load8<T>(x, beg + (gi << 3), v);
      group(v, beg + (gi << 3));
    }
    scalar_from = beg + (ngroups << 3);
  }
  for (int i = scalar_from + threadIdx.x; i < end; i += kThreads) {
    const float v = load1(x, i);
    if (v > m) {
      z *= fast_exp2((m - v) * c);
      m = v;
      a = i;
    }
    z += fast_exp2((v - m) * c);
  }
  // fixed-shape tree: wave (xor shuffles), then the four waves in order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float z2 = __shfl_xor(z, off);
    const int a2 = __shfl_xor(a, off);
    merge(m, z, a, m2, z2, a2, c);
  }
  __shared__ RowPart wave_part[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wave_part[wave] = RowPart{m, z, a, 0};
  __syncthreads();
  if (threadIdx.x == 0) {
    RowPart r = wave_part[0];
    for (int w = 1; w < kThreads / 64; ++w)
      merge(r.m, r.z, r.arg, wave_part[w].m, wave_part[w].z, wave_part[w].arg, c);
    part[static_cast<int64_t>(row) * splits + split] = r;
  }
}

// ------------------------------------------------------------- sampling
// Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds of two
// 32x32->64-bit products; the key advances by the Weyl constants between
// rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Noise stream of one slot: key = seed (low word first), counter =
// (token / 4, b * S + s, step, block), word token % 4.
struct NoiseKey {
  uint32_t k0, k1, row, step, block;
};

__device__ __forceinline__ uint32_t noise_word(const NoiseKey& nk, int v) {
  const uint4 w = philox4x32_10(make_uint4(static_cast<uint32_t>(v) >> 2, nk.row, nk.step, nk.block),
                                nk.k0, nk.k1);
  const int j = v & 3;
  return j == 0 ? w.x : (j == 1 ? w.y : (j == 2 ? w.z : w.w));
}

// Standard Gumbel draw from one word: u = (2 (w >> 9) + 1) 2^-24 (23 bits,
// strictly inside (0, 1), exact in fp32 and fp64), G = -ln(-ln u).  G lies in
// [-2.8117, 16.6356]; kGumbelLo/Hi bound that range with room to spare.
__device__ __forceinline__ float gumbel32(uint32_t w) {
  const float u = static_cast<float>(2u * (w >> 9) + 1u) * 5.9604644775390625e-08f;
  return -logf(-logf(u));
}
__device__ __forceinline__ double gumbel64(uint32_t w) {
  const double u = static_cast<double>(2u * (w >> 9) + 1u) * 5.9604644775390625e-08;
  return -log(-log(u));
}
constexpr float kGumbelSpread = 20.f;   // >= (kGumbelHi = 17) - (kGumbelLo = -3)

// Tokens whose logit is below m - cand_margin(m, tau) cannot reach within
// the decision band of the best perturbed score l + tau G of their slice
// (their score is at most l + 17 tau, the slice maximum's at least m - 3 tau):
// only the others draw noise.  The 2^-12 term keeps every token within
// kKeyBand * (1 + |m| + 20 tau) of the best score a candidate.
__device__ __forceinline__ float cand_margin(float m, float tau) {
  return kGumbelSpread * tau + 2.44140625e-04f * (1.f + fabsf(m));
}

struct SamplePart {
  float m;      // slice maximum
  float z;      // sum of exp2((x - m) * c) over the slice
  float key;    // best perturbed score l + tau G among the slice's candidates
  float key2;   // second best (-inf if none)
  int idx;      // token of `key` (INT_MAX if no candidate)
  float lx;     // its logit
  int pad0, pad1;
};

// (key, key2, idx, lx) <- the better of itself and (ok, ok2, oi, ol): higher
// score, lower token on equal scores; the second best follows.
__device__ __forceinline__ void merge_best(float& key, float& key2, int& idx, float& lx, float ok,
                                           float ok2, int oi, float ol) {
  if (ok > key || (ok == key && oi < idx)) {
    key2 = fmaxf(key, ok2);
    key = ok;
    idx = oi;
    lx = ol;
  } else {
    key2 = fmaxf(key2, ok);
  }
}

constexpr int kChunk = 8192;                   // tokens per workgroup pass
constexpr int kPerThread = kChunk / kThreads;  // 32: 4 groups of 8 consecutive tokens

// One pass's 32 logits per thread, kept as loaded: group u holds tokens
// base + 8 (tid + 256 u) .. + 7.  Tokens at or past `end` read as -inf.
template <typename T>
struct Chunk;

template <>
struct Chunk<uint16_t> {
  uint4 r[4];
  // a whole pass of 16-byte aligned tokens: unconditional loads, no branch
  __device__ __forceinline__ void load_full(const uint16_t* x, int base) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      r[u] = *reinterpret_cast<const uint4*>(x + base + 8 * (static_cast<int>(threadIdx.x) + kThreads * u));
  }
  __device__ __forceinline__ void load(const uint16_t* x, int base, int end, int vec_ok) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = base + 8 * (static_cast<int>(threadIdx.x) + kThreads * u);
      if (vec_ok && g + 8 <= end) {
        r[u] = *reinterpret_cast<const uint4*>(x + g);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = g + 2 * k < end ? x[g + 2 * k] : 0xff80u;
          const uint32_t hi = g + 2 * k + 1 < end ? x[g + 2 * k + 1] : 0xff80u;
          w[k] = lo | (hi << 16);
        }
        r[u] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
  __device__ __forceinline__ float get(int i) const {
    const uint4 q = r[i >> 3];
    const int k = i & 7;
    const uint32_t w = (k >> 1) == 0 ? q.x : ((k >> 1) == 1 ? q.y : ((k >> 1) == 2 ? q.z : q.w));
    return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};

template <>
struct Chunk<float> {
  float4 r[8];
  __device__ __forceinline__ void load_full(const float* x, int base) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = base + 8 * (static_cast<int>(threadIdx.x) + kThreads * u);
      r[2 * u] = *reinterpret_cast<const float4*>(x + g);
      r[2 * u + 1] = *reinterpret_cast<const float4*>(x + g + 4);
    }
  }
  __device__ __forceinline__ void load(const float* x, int base, int end, int vec_ok) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = base + 8 * (static_cast<int>(threadIdx.x) + kThreads * u);
      if (vec_ok && g + 8 <= end) {
        r[2 * u] = *reinterpret_cast<const float4*>(x + g);
        r[2 * u + 1] = *reinterpret_cast<const float4*>(x + g + 4);
      } else {
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = g + k < end ? x[g + k] : -INFINITY;
        r[2 * u] = make_float4(w[0], w[1], w[2], w[3]);
        r[2 * u + 1] = make_float4(w[4], w[5], w[6], w[7]);
      }
    }
  }
  __device__ __forceinline__ float get(int i) const {
    const float4 q = r[i >> 2];
    const int k = i & 3;
    return k == 0 ? q.x : (k == 1 ? q.y : (k == 2 ? q.z : q.w));
  }
};

// Streams one slice [split*split_len, +split_len) of one masked row in passes
// of 8192 tokens, the next pass's loads in flight while the current one is
// processed (whole aligned passes; a partial or unaligned pass is loaded and
// processed on its own).  Per pass: the workgroup maximum (one barrier), the running
// reference M = max so far (Z rescaled when it grows), Z += exp2((x - M) c),
// and the Gumbel-max candidates x >= M - cand_margin(M): the token holding
// M was itself a candidate when it arrived, and it outscores every token
// left out, so the best perturbed score of the slice is among the candidates.
// (A running maximum per wave instead, with no barrier, was slower: the
// waves' maxima grow later, so more tokens pass as candidates.)
template <typename T>
__global__ __launch_bounds__(kThreads) void rowsample_kernel(
    const T* __restrict__ logits, int64_t row_stride, int V, const uint8_t* __restrict__ masked,
    float c, float tau, NoiseKey nk, int split_len, int splits, int vec_ok,
    SamplePart* __restrict__ part) {
  const int row = blockIdx.y;
  if (!masked[row]) return;
  const int split = blockIdx.x;
  const int beg = split * split_len;
  const int end = min(V, beg + split_len);
  const T* x = logits + static_cast<int64_t>(row) * row_stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  NoiseKey rk = nk;
  rk.row = static_cast<uint32_t>(row);
  __shared__ float s_cmax[2][kThreads / 64];
  __shared__ float s_red[kThreads / 64];
  __shared__ SamplePart s_best[kThreads / 64];
  float M = -FLT_MAX, z = 0.f;
  float key = -INFINITY, key2 = -INFINITY, lx = 0.f;
  int idx = INT_MAX;
  // one pass over the tokens a chunk holds (cb: its first token)
  int pass = 0;
  auto process = [&](const Chunk<T>& cur, int cb) {
    float tm = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) tm = fmaxf(tm, cur.get(i));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tm = fmaxf(tm, __shfl_xor(tm, off));
    // two slots, alternating: a slot is rewritten only after the next
    // barrier, which every thread passes after reading it
    if (lane == 0) s_cmax[pass & 1][wave] = tm;
    __syncthreads();
    const float C = fmaxf(fmaxf(s_cmax[pass & 1][0], s_cmax[pass & 1][1]),
                          fmaxf(s_cmax[pass & 1][2], s_cmax[pass & 1][3]));
    ++pass;
    if (C > M) {   // workgroup-uniform
      z *= fast_exp2((M - C) * c);
      M = C;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = fast_exp2((cur.get(8 * u + j) - M) * c);
      z += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    }
    // a bit per candidate, then one loop body for all of them; the logit is
    // picked out of the loaded registers by a select over the 32 slots (a
    // reload from memory made every pass with a candidate wait a full memory
    // round trip before the next barrier)
    const float thr = M - cand_margin(M, tau);
    uint32_t cand = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const float v = cur.get(i);
      cand |= (v >= thr && v != -INFINITY) ? (1u << i) : 0u;
    }
    while (cand) {
      const int i = __builtin_ctz(cand);
      cand &= cand - 1;
      const int t = cb + 8 * (tid + kThreads * (i >> 3)) + (i & 7);
      float l = 0.f;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) l = (k == i) ? cur.get(k) : l;
      const float sc = l + tau * gumbel32(noise_word(rk, t));
      merge_best(key, key2, idx, lx, sc, -INFINITY, t, l);
    }
  };
  // whole passes of 16-byte aligned tokens: two register buffers taken in
  // turn, the next pass's loads issued before the current pass is processed.
  // No copy between the buffers and no branch around a load (the last
  // pass's fetch repeats its own addresses, in bounds and unused): a copy or
  // a branchy load made the compiler wait for the next pass's loads before
  // processing the current one, so each pass paid a full memory round trip.
  const int nfull = vec_ok ? (end - beg) / kChunk : 0;
  if (nfull > 0) {
    Chunk<T> ca, cbf;
    ca.load_full(x, beg);
    for (int k = 0;;) {
      cbf.load_full(x, beg + (k + 1 < nfull ? k + 1 : k) * kChunk);
      process(ca, beg + k * kChunk);
      if (++k == nfull) break;
      ca.load_full(x, beg + (k + 1 < nfull ? k + 1 : k) * kChunk);
      process(cbf, beg + k * kChunk);
      if (++k == nfull) break;
    }
  }
  // the rest: a partial last pass, or every pass of a row whose tokens are
  // not 16-byte aligned (tokens at or past `end` read as -inf)
  for (int cb = beg + nfull * kChunk; cb < end; cb += kChunk) {
    Chunk<T> cur;
    cur.load(x, cb, end, vec_ok);
    process(cur, cb);
  }
  // fixed-shape trees: Z and the best pair over the wave, then the four waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    z += __shfl_xor(z, off);
    const float ok = __shfl_xor(key, off), ok2 = __shfl_xor(key2, off), ol = __shfl_xor(lx, off);
    const int oi = __shfl_xor(idx, off);
    merge_best(key, key2, idx, lx, ok, ok2, oi, ol);
  }
  if (lane == 0) {
    s_red[wave] = z;
    s_best[wave] = SamplePart{M, z, key, key2, idx, lx, 0, 0};
  }
  __syncthreads();
  if (tid == 0) {
    SamplePart r = s_best[0];
    r.z = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    for (int w = 1; w < kThreads / 64; ++w)
      merge_best(r.key, r.key2, r.idx, r.lx, s_best[w].key, s_best[w].key2, s_best[w].idx,
                 s_best[w].lx);
    part[static_cast<int64_t>(row) * splits + split] = r;
  }
}

// The decision kernel runs one workgroup per sequence; its fp64 full-row
// scans (rescoring near-tied Gumbel scores, rechecking confidences near a
// decision boundary) are reads of a whole row by that one workgroup, so it is
// a large one: 16 waves keep 64 KB of the row in flight.
constexpr int kDecideThreads = 1024;
constexpr int kPartBatch = 8;   // slice records loaded together per row

// fp64 rescoring of one row's candidates (those within cand_margin of the
// row maximum m): the token of the largest l + tau G in fp64, lowest token on
// equal scores.  All threads take part; every thread returns the result.
template <typename T>
__device__ void rescore_row64(const T* x, int V, float m, float tau, double tau64, const NoiseKey& nk,
                              double* red_k, int* red_i, int& out_idx, float& out_l) {
  const float thr = m - cand_margin(m, tau);
  double best = -INFINITY;
  int bi = INT_MAX;
  auto visit = [&](float l, int t) {
    if (l >= thr && l != -INFINITY) {
      const double sc = static_cast<double>(l) + tau64 * gumbel64(noise_word(nk, t));
      if (sc > best || (sc == best && t < bi)) {
        best = sc;
        bi = t;
      }
    }
  };
  // scalar head up to 16-byte alignment, then groups of 8 logits (four
  // 16-byte loads in flight per thread: the scan is a full read of the row),
  // then a scalar tail
  const int head = min(V, static_cast<int>(((16 - reinterpret_cast<uintptr_t>(x) % 16) % 16) / sizeof(T)));
  if (static_cast<int>(threadIdx.x) < head) visit(load1(x, threadIdx.x), threadIdx.x);
  const int nvec = (V - head) / 8;
  int j = threadIdx.x;
  for (; j + 3 * kDecideThreads < nvec; j += 4 * kDecideThreads) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(x, head + 8 * static_cast<int64_t>(j + u * kDecideThreads), v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float g = fmaxf(fmaxf(fmaxf(v[u][0], v[u][1]), fmaxf(v[u][2], v[u][3])),
                      fmaxf(fmaxf(v[u][4], v[u][5]), fmaxf(v[u][6], v[u][7])));
      if (g >= thr)
        for (int k = 0; k < 8; ++k) visit(v[u][k], head + 8 * (j + u * kDecideThreads) + k);
    }
  }
  for (; j < nvec; j += kDecideThreads) {
    float v[8];
    load8<T>(x, head + 8 * static_cast<int64_t>(j), v);
    for (int k = 0; k < 8; ++k) visit(v[k], head + 8 * j + k);
  }
  for (int t = head + 8 * nvec + threadIdx.x; t < V; t += kDecideThreads) visit(load1(x, t), t);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    red_k[wave] = best;
    red_i[wave] = bi;
  }
  __syncthreads();
  best = red_k[0];
  bi = red_i[0];
  for (int w = 1; w < kDecideThreads / 64; ++w)
    if (red_k[w] > best || (red_k[w] == best && red_i[w] < bi)) {
      best = red_k[w];
      bi = red_i[w];
    }
  __syncthreads();
  if (bi == INT_MAX) bi = 0;   // no finite logit: outside the contract
  out_idx = bi;
  out_l = load1(x, bi);
}

// fp64 probability of the argmax of one row: 1 / sum_v exp((x_v - m) / tau),
// reduced in a fixed order (thread-strided sums, then a fixed tree) so equal
// rows give equal bits.
template <typename T>
__device__ double recheck_row(const T* x, int V, float m, double tau, double* red) {
  double acc = 0.0;
  const double md = static_cast<double>(m);
  const double inv = 1.0 / tau;
  // Terms with (l - m)/tau < -50 are left out: each is below e^-50 of the
  // largest term (1), so all of them together move Z by less than
  // V e^-50 < 3e-17 relative at V = 2^17, under fp64 rounding.  The
  // exponential runs only where some lane of the wave needs it: at low
  // temperature a handful of terms per row.
  auto term = [&](float v) {
    const double a = (static_cast<double>(v) - md) * inv;
    return a > -50.0 ? exp(a) : 0.0;
  };
  // scalar head up to 16-byte alignment, then groups of 8 logits with four
  // groups' loads in flight per thread (the scan is a full read of the row
  // by one workgroup: one load at a time left it waiting on memory), then
  // the remaining groups and a scalar tail
  const int head = min(V, static_cast<int>(((16 - reinterpret_cast<uintptr_t>(x) % 16) % 16) / sizeof(T)));
  if (static_cast<int>(threadIdx.x) < head) acc += term(load1(x, threadIdx.x));
  const int nvec = (V - head) / 8;
  auto group = [&](const float (&v)[8]) {
    double s8 = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double a = (static_cast<double>(v[k]) - md) * inv;
      if (a > -50.0) s8 += exp(a);
    }
    acc += s8;
  };
  int j = threadIdx.x;
  for (; j + 3 * kDecideThreads < nvec; j += 4 * kDecideThreads) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(x, head + 8 * static_cast<int64_t>(j + u * kDecideThreads), v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) group(v[u]);
  }
  for (; j < nvec; j += kDecideThreads) {
    float v[8];
    load8<T>(x, head + 8 * static_cast<int64_t>(j), v);
    group(v);
  }
  for (int i = head + 8 * nvec + threadIdx.x; i < V; i += kDecideThreads) acc += term(load1(x, i));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  double t[kDecideThreads / 64];
#pragma unroll
  for (int w = 0; w < kDecideThreads / 64; ++w) t[w] = red[w];
#pragma unroll
  for (int h = kDecideThreads / 128; h >= 1; h >>= 1)   // fixed pairwise tree
#pragma unroll
    for (int w = 0; w < h; ++w) t[w] += t[w + h];
  __syncthreads();
  return 1.0 / t[0];
}

template <typename T, bool SAMPLE>
__global__ __launch_bounds__(kDecideThreads) void decide_kernel(
    const T* __restrict__ logits, int64_t row_stride, int S, int V,
    const void* __restrict__ parts, int splits, float c, float gamma, float tau, double tau64,
    NoiseKey nk, int mask_id, int step, int32_t* tokens, uint8_t* masked, uint8_t* committed_now,
    float* conf, int32_t* pred, int8_t* commit_step, int32_t* n_masked) {
  __shared__ float s_m[64];
  __shared__ float s_lx[64];      // logit of the prediction (= s_m for the argmax)
  __shared__ float s_z[64];       // fp32 Z relative to s_m (sampling)
  __shared__ int s_pred[64];
  __shared__ double s_p[64];      // fp32 p widened, or the fp64 recheck
  __shared__ int s_checked[64];
  __shared__ int s_msk[64];
  __shared__ int s_rescore[64];
  __shared__ double red[kDecideThreads / 64];
  __shared__ int red_i[kDecideThreads / 64];
  __shared__ int s_choice;        // -1: threshold set; else the single slot
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(b) * S;
  if (tid < S) {
    const int msk = masked[row0 + tid] != 0;
    s_msk[tid] = msk;
    s_checked[tid] = 0;
    s_rescore[tid] = 0;
    // The slice records are loaded kPartBatch at a time (the loads of a
    // batch in flight together; indices past the last slice re-read it and
    // are ignored) and folded in slice order as one by one: one memory round
    // trip per batch instead of one per slice (32 slices per row for a
    // single sequence).
    if (msk && !SAMPLE) {
      const RowPart* p = static_cast<const RowPart*>(parts) + (row0 + tid) * splits;
      float m = 0.f, z = 0.f;
      int a = INT_MAX;
      for (int k0 = 0; k0 < splits; k0 += kPartBatch) {
        RowPart q[kPartBatch];
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j) q[j] = p[min(k0 + j, splits - 1)];
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j) {
          if (k0 + j == 0) {
            m = q[j].m;
            z = q[j].z;
            a = q[j].arg;
          } else if (k0 + j < splits) {
            merge(m, z, a, q[j].m, q[j].z, q[j].arg, c);
          }
        }
      }
      s_m[tid] = m;
      s_lx[tid] = m;
      s_pred[tid] = a;
      s_p[tid] = static_cast<double>(1.0f / z);
    } else if (msk) {
      // slices in order: row maximum, Z relative to it, best perturbed score
      const SamplePart* p = static_cast<const SamplePart*>(parts) + (row0 + tid) * splits;
      float m = -INFINITY;
      for (int k0 = 0; k0 < splits; k0 += kPartBatch) {
        float mk[kPartBatch];
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j) mk[j] = p[min(k0 + j, splits - 1)].m;
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j)
          if (k0 + j < splits) m = k0 + j == 0 ? mk[j] : fmaxf(m, mk[j]);
      }
      float z = 0.f, key = 0.f, key2 = 0.f, lx = 0.f;
      int idx = INT_MAX;
      for (int k0 = 0; k0 < splits; k0 += kPartBatch) {
        SamplePart q[kPartBatch];
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j) q[j] = p[min(k0 + j, splits - 1)];
#pragma unroll
        for (int j = 0; j < kPartBatch; ++j) {
          const int k = k0 + j;
          if (k >= splits) continue;
          z += q[j].z * fast_exp2((q[j].m - m) * c);
          if (k == 0) {
            key = q[j].key;
            key2 = q[j].key2;
            idx = q[j].idx;
            lx = q[j].lx;
          } else {
            merge_best(key, key2, idx, lx, q[j].key, q[j].key2, q[j].idx, q[j].lx);
          }
        }
      }
      s_m[tid] = m;
      s_z[tid] = z;
      s_lx[tid] = lx;
      s_pred[tid] = idx;
      s_p[tid] = static_cast<double>(fast_exp2((lx - m) * c) / z);
      // the fp32 scores of the two best can be off by far less than this band
      s_rescore[tid] = (key - key2) <= kKeyBand * (1.f + fabsf(m) + kGumbelSpread * tau);
    }
  }
  __syncthreads();
  if (SAMPLE) {
    // near-ties of the perturbed scores: rescore the row's candidates in fp64
    for (int s = 0; s < S; ++s) {
      if (s_msk[s] && s_rescore[s]) {
        NoiseKey k = nk;
        k.row = static_cast<uint32_t>(row0 + s);
        int idx;
        float lx;
        rescore_row64<T>(logits + (row0 + s) * row_stride, V, s_m[s], tau, tau64, k, red, red_i,
                         idx, lx);
        if (tid == 0) {
          s_pred[s] = idx;
          s_lx[s] = lx;
          s_p[s] = static_cast<double>(fast_exp2((lx - s_m[s]) * c) / s_z[s]);
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
  // rows whose fp32 p is within kDelta of gamma: decide them in fp64
  for (int s = 0; s < S; ++s) {
    if (s_msk[s] && fabs(s_p[s] - static_cast<double>(gamma)) <= kDelta) {
      const double p64 = exp((static_cast<double>(s_lx[s]) - s_m[s]) / tau64) *
                         recheck_row<T>(logits + (row0 + s) * row_stride, V, s_m[s], tau64, red);
      if (tid == 0) { s_p[s] = p64; s_checked[s] = 1; }
      __syncthreads();
    }
  }
  if (tid == 0) {
    int any_pass = 0, any_masked = 0;
    double best = -1.0;
    for (int s = 0; s < S; ++s) {
      if (!s_msk[s]) continue;
      any_masked = 1;
      if (s_p[s] >= static_cast<double>(gamma)) any_pass = 1;
      best = fmax(best, s_p[s]);
    }
    s_choice = -1;
    red[0] = best;
    if (!any_pass && any_masked) s_choice = -2;  // one-commit rule applies
  }
  __syncthreads();
  if (s_choice == -2) {
    // every row within 2*kDelta of the best fp32/fp64 p is settled in fp64 --
    // unless the best is the only such row: every p is within kDelta/10 of
    // its fp64 value, so the fp64 argmax is then that same row
    const double best = red[0];
    __syncthreads();
    int near = 0;
    for (int s = 0; s < S; ++s) near += s_msk[s] && s_p[s] >= best - 2.0 * kDelta;
    for (int s = 0; s < S && near > 1; ++s) {
      if (s_msk[s] && !s_checked[s] && s_p[s] >= best - 2.0 * kDelta) {
        const double p64 = exp((static_cast<double>(s_lx[s]) - s_m[s]) / tau64) *
                           recheck_row<T>(logits + (row0 + s) * row_stride, V, s_m[s], tau64, red);
        if (tid == 0) { s_p[s] = p64; s_checked[s] = 1; }
        __syncthreads();
      }
    }
    if (tid == 0) {
      int top = -1;
      for (int s = 0; s < S; ++s)
        if (s_msk[s] && (top < 0 || s_p[s] > s_p[top])) top = s;  // lowest s on ties
      s_choice = top;
    }
    __syncthreads();
  }
  if (tid < 64) {
    const int s = tid;
    int remaining = 0;
    if (s < S) {
      const int64_t r = row0 + s;
      if (s_msk[s]) {
        const int take = (s_choice == -1) ? (s_p[s] >= static_cast<double>(gamma)) : (s == s_choice);
        tokens[r] = take ? s_pred[s] : mask_id;
        masked[r] = take ? 0 : 1;
        remaining = !take;
        if (committed_now) committed_now[r] = take;
        if (conf) conf[r] = static_cast<float>(s_p[s]);
        if (pred) pred[r] = s_pred[s];
        if (commit_step && take) commit_step[r] = static_cast<int8_t>(step);
      } else {
        if (committed_now) committed_now[r] = 0;
        if (conf) conf[r] = __builtin_nanf("");
        if (pred) pred[r] = -1;
      }
    }
    const unsigned long long bal = __ballot(remaining);
    if (s == 0 && n_masked) n_masked[b] = __popcll(bal);
  }
}

}  // namespace

UnmaskPlan unmask_plan(int B, int S, int V) {
  UnmaskPlan p{};
  const int64_t rows = static_cast<int64_t>(B) * S;
  int splits = static_cast<int>(ceil_div(2 * device_cus(), rows));
  splits = splits < 1 ? 1 : (splits > 64 ? 64 : splits);
  int64_t len = align_up(static_cast<size_t>(ceil_div(V, splits)), 8);
  if (len < 2048) len = 2048;
  p.split_len = static_cast<int>(len);
  p.splits = static_cast<int>(ceil_div(V, len));
  p.s_splits = p.splits;   // the sampling pass streams the same slices
  p.part_bytes = align_up(static_cast<size_t>(rows) * p.splits * sizeof(RowPart), 256);
  p.s_part_bytes = align_up(static_cast<size_t>(rows) * p.s_splits * sizeof(SamplePart), 256);
  p.total_bytes = p.part_bytes > p.s_part_bytes ? p.part_bytes : p.s_part_bytes;
  return p;
}

namespace {

template <typename T>
void launch_unmask_t(const UnmaskArgs& a, const UnmaskPlan& p, void* ws, int vec, hipStream_t st) {
  const T* x = static_cast<const T*>(a.logits);
  const float c = static_cast<float>(1.4426950408889634 / static_cast<double>(a.temperature));
  const double tau64 = static_cast<double>(a.temperature);
  NoiseKey nk{static_cast<uint32_t>(a.seed & 0xffffffffu), static_cast<uint32_t>(a.seed >> 32), 0u,
              static_cast<uint32_t>(a.step), static_cast<uint32_t>(a.block_index)};
  const dim3 blk(kThreads);
  if (!a.sample) {
    RowPart* part = static_cast<RowPart*>(ws);
    hipLaunchKernelGGL(rowreduce_kernel<T>, dim3(p.splits, a.B * a.S), blk, 0, st, x, a.row_stride,
                       a.V, a.masked, c, p.split_len, p.splits, vec, part);
    hipLaunchKernelGGL((decide_kernel<T, false>), dim3(a.B), dim3(kDecideThreads), 0, st, x, a.row_stride, a.S, a.V,
                       static_cast<const void*>(part), p.splits, c, a.gamma, a.temperature, tau64,
                       nk, a.mask_id, a.step, a.tokens, a.masked, a.committed_now, a.conf, a.pred,
                       a.commit_step, a.n_masked);
  } else {
    SamplePart* part = static_cast<SamplePart*>(ws);
    hipLaunchKernelGGL(rowsample_kernel<T>, dim3(p.s_splits, a.B * a.S), blk, 0, st, x,
                       a.row_stride, a.V, a.masked, c, a.temperature, nk, p.split_len, p.s_splits,
                       vec, part);
    hipLaunchKernelGGL((decide_kernel<T, true>), dim3(a.B), dim3(kDecideThreads), 0, st, x, a.row_stride, a.S, a.V,
                       static_cast<const void*>(part), p.s_splits, c, a.gamma, a.temperature,
                       tau64, nk, a.mask_id, a.step, a.tokens, a.masked, a.committed_now, a.conf,
                       a.pred, a.commit_step, a.n_masked);
  }
}

}  // namespace

hipError_t launch_confidence_unmask(const UnmaskArgs& a, const UnmaskPlan& p, void* ws,
                                    hipStream_t st) {
  if (a.dtype == 0) {
    const int vec = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) && (a.row_stride % 8 == 0);
    launch_unmask_t<uint16_t>(a, p, ws, vec, st);
  } else {
    const int vec = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) && (a.row_stride % 4 == 0);
    launch_unmask_t<float>(a, p, ws, vec, st);
  }
  return hipGetLastError();
}

}  // namespace tt
