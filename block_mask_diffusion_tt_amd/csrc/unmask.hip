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
#include <float.h>
#include <limits.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kThreads = 256;
constexpr float kDelta = 6.103515625e-05f;  // 2^-14

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
    // four 16-byte loads in flight per thread, consumed in index order
    for (; gi + 3 * kThreads < ngroups; gi += 4 * kThreads) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8<T>(x, beg + ((gi + u * kThreads) << 3), v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) group(v[u], beg + ((gi + u * kThreads) << 3));
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

// fp64 probability of the argmax of one row: 1 / sum_v exp((x_v - m) / tau),
// reduced in a fixed order (thread-strided sums, then a fixed tree) so equal
// rows give equal bits.
template <typename T>
__device__ double recheck_row(const T* x, int V, float m, double tau, double* red) {
  double acc = 0.0;
  const double md = static_cast<double>(m);
  // scalar head up to 16-byte alignment, then 8 logits per thread per
  // iteration (one or two 16-byte loads, eight independent exponentials),
  // then a scalar tail
  const int head = min(V, static_cast<int>(((16 - reinterpret_cast<uintptr_t>(x) % 16) % 16) / sizeof(T)));
  if (static_cast<int>(threadIdx.x) < head)
    acc += exp((static_cast<double>(load1(x, threadIdx.x)) - md) / tau);
  const int nvec = (V - head) / 8;
  for (int j = threadIdx.x; j < nvec; j += kThreads) {
    float v[8];
    load8<T>(x, head + 8 * static_cast<int64_t>(j), v);
    double e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = exp((static_cast<double>(v[k]) - md) / tau);
    acc += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }
  for (int i = head + 8 * nvec + threadIdx.x; i < V; i += kThreads)
    acc += exp((static_cast<double>(load1(x, i)) - md) / tau);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  double tot = ((red[0] + red[1]) + (red[2] + red[3]));
  __syncthreads();
  return 1.0 / tot;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void decide_kernel(
    const T* __restrict__ logits, int64_t row_stride, int S, int V,
    const RowPart* __restrict__ part, int splits, float c, float gamma, double tau,
    int mask_id, int step, int32_t* tokens, uint8_t* masked, uint8_t* committed_now,
    float* conf, int32_t* pred, int8_t* commit_step, int32_t* n_masked) {
  __shared__ float s_m[64];
  __shared__ int s_pred[64];
  __shared__ double s_p[64];      // fp32 p widened, or the fp64 recheck
  __shared__ int s_checked[64];
  __shared__ int s_msk[64];
  __shared__ double red[kThreads / 64];
  __shared__ int s_choice;        // -1: threshold set; else the single slot
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(b) * S;
  if (tid < S) {
    const int msk = masked[row0 + tid] != 0;
    s_msk[tid] = msk;
    s_checked[tid] = 0;
    if (msk) {
      const RowPart* p = part + (row0 + tid) * splits;
      float m = p[0].m, z = p[0].z;
      int a = p[0].arg;
      for (int k = 1; k < splits; ++k) merge(m, z, a, p[k].m, p[k].z, p[k].arg, c);
      s_m[tid] = m;
      s_pred[tid] = a;
      s_p[tid] = static_cast<double>(1.0f / z);
    }
  }
  __syncthreads();
  // rows whose fp32 p is within kDelta of gamma: decide them in fp64
  for (int s = 0; s < S; ++s) {
    if (s_msk[s] && fabs(s_p[s] - static_cast<double>(gamma)) <= kDelta) {
      const double p64 = recheck_row<T>(logits + (row0 + s) * row_stride, V, s_m[s], tau, red);
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
        const double p64 = recheck_row<T>(logits + (row0 + s) * row_stride, V, s_m[s], tau, red);
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
  int splits = static_cast<int>(ceil_div(2 * kNumCUs, rows));
  splits = splits < 1 ? 1 : (splits > 64 ? 64 : splits);
  int64_t len = align_up(static_cast<size_t>(ceil_div(V, splits)), 8);
  if (len < 2048) len = 2048;
  p.split_len = static_cast<int>(len);
  p.splits = static_cast<int>(ceil_div(V, len));
  p.part_bytes = align_up(static_cast<size_t>(rows) * p.splits * sizeof(RowPart), 256);
  p.total_bytes = p.part_bytes;
  return p;
}

hipError_t launch_confidence_unmask(const UnmaskArgs& a, const UnmaskPlan& p, void* ws,
                                    hipStream_t st) {
  RowPart* part = static_cast<RowPart*>(ws);
  const float c = static_cast<float>(1.4426950408889634 / static_cast<double>(a.temperature));
  const double tau = static_cast<double>(a.temperature);
  const dim3 g1(p.splits, a.B * a.S), blk(kThreads);
  if (a.dtype == 0) {
    const auto* x = static_cast<const uint16_t*>(a.logits);
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (a.row_stride % 8 == 0);
    hipLaunchKernelGGL(rowreduce_kernel<uint16_t>, g1, blk, 0, st, x, a.row_stride, a.V, a.masked,
                       c, p.split_len, p.splits, vec, part);
    hipLaunchKernelGGL(decide_kernel<uint16_t>, dim3(a.B), blk, 0, st, x, a.row_stride, a.S, a.V,
                       part, p.splits, c, a.gamma, tau, a.mask_id, a.step, a.tokens, a.masked,
                       a.committed_now, a.conf, a.pred, a.commit_step, a.n_masked);
  } else {
    const auto* x = static_cast<const float*>(a.logits);
    const int vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (a.row_stride % 4 == 0);
    hipLaunchKernelGGL(rowreduce_kernel<float>, g1, blk, 0, st, x, a.row_stride, a.V, a.masked, c,
                       p.split_len, p.splits, vec, part);
    hipLaunchKernelGGL(decide_kernel<float>, dim3(a.B), blk, 0, st, x, a.row_stride, a.S, a.V,
                       part, p.splits, c, a.gamma, tau, a.mask_id, a.step, a.tokens, a.masked,
                       a.committed_now, a.conf, a.pred, a.commit_step, a.n_masked);
  }
  return hipGetLastError();
}

}  // namespace tt
