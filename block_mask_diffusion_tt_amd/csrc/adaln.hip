// Timestep conditioning (adaLN-single) and the small bookkeeping kernels of
// the denoising loop.
//
// [dothoosh] two-tower mechanism section: every denoiser layer is modulated
// by the diffusion timestep through adaLN-single, about 1.5 M parameters.
// [modelcard] technical features section: scale, shift and gate are injected
// per timestep into each layer.  The embedding (DiT sinusoid), the shared
// SiLU -> Linear(256 -> 3*width) and the per-layer table are the reading of
// "adaLN-single" used throughout (PixArt-alpha's construction).
#include <math.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kEmb = 256;

// emb[b, i] = cos(1000 t f_i), emb[b, 128 + i] = sin(1000 t f_i),
// f_i = 10000^(-i/128); t from `t` or, when t is NULL, n_masked[b] / S.
__global__ void timestep_embed_kernel(int B, const float* t, const int32_t* n_masked, int S,
                                      float* emb) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;  // 0..127
  if (b >= B || i >= kEmb / 2) return;
  const double tb = t ? static_cast<double>(t[b])
                      : static_cast<double>(n_masked[b]) / static_cast<double>(S);
  const double f = exp(-log(10000.0) * static_cast<double>(i) / (kEmb / 2));
  const double arg = 1000.0 * tb * f;
  double sn, cs;
  sincos(arg, &sn, &cs);
  emb[static_cast<int64_t>(b) * kEmb + i] = static_cast<float>(cs);
  emb[static_cast<int64_t>(b) * kEmb + kEmb / 2 + i] = static_cast<float>(sn);
}

// u = SiLU(emb) @ W for a tile of kRows sequences x 128 columns per
// workgroup: 256 threads = 8 k-slices x 32 column quads.  Each thread owns 4
// adjacent columns for the tile's rows and 32 values of k; its 32 loads of W
// (8 bytes each) are issued before any arithmetic.  The 8 k-slices are summed
// in LDS in a fixed order (deterministic), then the epilogue adds the bias and
// writes every layer's copy with its table row.
constexpr int kRows = 8;   // 16 rows halve the W re-reads but their LDS allows one
                           // workgroup per CU: twice as slow, measured
constexpr int kCols = 128;
constexpr int kSlices = 8;
constexpr int kPerSlice = kEmb / kSlices;

__global__ __launch_bounds__(256) void adaln_kernel(int B, int width, int n_layers,
                                                    const float* __restrict__ emb,
                                                    const uint16_t* __restrict__ w,
                                                    const float* __restrict__ bias,
                                                    const float* __restrict__ table,
                                                    float* __restrict__ ada) {
  __shared__ float s_e[kRows][kEmb];
  __shared__ float s_part[kSlices][kRows][kCols + 4];
  const int N = 3 * width;
  const int n0 = blockIdx.x * kCols;
  const int b0 = blockIdx.y * kRows;
  const int nb = min(kRows, B - b0);
  const int slice = threadIdx.x >> 5, cq = threadIdx.x & 31;
  const int n = n0 + 4 * cq;
  uint2 wv[kPerSlice];
  if (n < N) {   // width is a multiple of 4, so a quad never straddles N
    const uint16_t* wp = w + static_cast<int64_t>(slice * kPerSlice) * N + n;
#pragma unroll
    for (int kk = 0; kk < kPerSlice; ++kk)
      wv[kk] = *reinterpret_cast<const uint2*>(wp + static_cast<int64_t>(kk) * N);
  } else {
#pragma unroll
    for (int kk = 0; kk < kPerSlice; ++kk) wv[kk] = make_uint2(0, 0);
  }
  // SiLU of the tile's embeddings into LDS: every load issued before the
  // first use (one round trip)
  constexpr int kEPer = kRows * kEmb / 256;
  float ev[kEPer];
#pragma unroll
  for (int i = 0; i < kEPer; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int r = idx / kEmb, k = idx % kEmb;
    ev[i] = r < nb ? emb[static_cast<int64_t>(b0 + r) * kEmb + k] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kEPer; ++i) {
    const int idx = threadIdx.x + 256 * i;
    s_e[idx / kEmb][idx % kEmb] = ev[i] / (1.f + expf(-ev[i]));
  }
  __syncthreads();
  float acc[kRows][4];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[r][j] = 0.f;
#pragma unroll
  for (int kk = 0; kk < kPerSlice; kk += 4) {
    float wf[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wf[q][0] = __uint_as_float(wv[kk + q].x << 16);
      wf[q][1] = __uint_as_float(wv[kk + q].x & 0xffff0000u);
      wf[q][2] = __uint_as_float(wv[kk + q].y << 16);
      wf[q][3] = __uint_as_float(wv[kk + q].y & 0xffff0000u);
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const float4 e = *reinterpret_cast<const float4*>(&s_e[r][slice * kPerSlice + kk]);
      const float ev[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[r][j] = fmaf(ev[q], wf[q][j], acc[r][j]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_part[slice][r][4 * cq + j] = acc[r][j];
  __syncthreads();
  // epilogue: one 4-column quad of one row per thread and pass (8 rows x 32
  // quads per pass); width is a multiple of 4, so a quad never straddles
  // shift/scale/gate
  for (int r = threadIdx.x >> 5; r < kRows; r += 256 / 32) {
    const int q = threadIdx.x & 31;
    const int col = n0 + 4 * q;
    if (r < nb && col < N) {
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) {
        const float4 v = *reinterpret_cast<const float4*>(&s_part[sl][r][4 * q]);
        u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
      }
      if (bias) {
        const float4 bv = *reinterpret_cast<const float4*>(bias + col);
        u.x += bv.x; u.y += bv.y; u.z += bv.z; u.w += bv.w;
      }
      const int j = col / width, cc = col % width;
      for (int l = 0; l < n_layers; ++l) {
        float4 o = u;
        if (table) {
          const float4 tv = *reinterpret_cast<const float4*>(table + (static_cast<int64_t>(l) * 3 + j) * width + cc);
          o.x += tv.x; o.y += tv.y; o.z += tv.z; o.w += tv.w;
        }
        *reinterpret_cast<float4*>(ada + ((static_cast<int64_t>(l) * 3 + j) * B + b0 + r) * width + cc) = o;
      }
    }
  }
}

__global__ void active_kernel(int B, const int32_t* n_masked, uint8_t* active, int32_t* total) {
  int local = 0;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int n = n_masked[b];
    active[b] = n > 0;
    local += n;
  }
  for (int off = 32; off >= 1; off >>= 1) local += __shfl_xor(local, off);
  __shared__ int s[16];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < static_cast<int>(blockDim.x >> 6); ++i) t += s[i];
    *total = t;
  }
}

__global__ void count_masked_kernel(int B, int S, const uint8_t* masked, int32_t* n_masked) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = 0;
  for (int s = 0; s < S; ++s) n += masked[static_cast<int64_t>(b) * S + s] != 0;
  n_masked[b] = n;
}

__global__ void clear_kernel(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t k = i; k < n16; k += stride) p[k] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

}  // namespace

hipError_t launch_timestep_embed(int B, const float* t, const int32_t* n_masked, int S,
                                 float* emb, hipStream_t st) {
  hipLaunchKernelGGL(timestep_embed_kernel, dim3(B), dim3(kEmb / 2), 0, st, B, t, n_masked, S, emb);
  return hipGetLastError();
}

hipError_t launch_adaln_single(int B, int width, int n_layers, const float* emb, const void* w,
                               const float* bias, const float* table, float* ada,
                               hipStream_t st) {
  const int N = 3 * width;
  const dim3 grid(static_cast<unsigned>(ceil_div(N, kCols)), static_cast<unsigned>(ceil_div(B, kRows)));
  hipLaunchKernelGGL(adaln_kernel, grid, dim3(256), 0, st, B, width, n_layers, emb,
                     static_cast<const uint16_t*>(w), bias, table, ada);
  return hipGetLastError();
}

hipError_t launch_active_from_masked(int B, const int32_t* n_masked, uint8_t* active,
                                     int32_t* total, hipStream_t st) {
  hipLaunchKernelGGL(active_kernel, dim3(1), dim3(1024), 0, st, B, n_masked, active, total);
  return hipGetLastError();
}

hipError_t launch_count_masked(int B, int S, const uint8_t* masked, int32_t* n_masked,
                               hipStream_t st) {
  hipLaunchKernelGGL(count_masked_kernel, dim3(static_cast<unsigned>(ceil_div(B, 256))), dim3(256),
                     0, st, B, S, masked, n_masked);
  return hipGetLastError();
}

hipError_t launch_clear(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  uint8_t* tail = static_cast<uint8_t*>(p) + n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(clear_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<uint4*>(p), n16, tail, ntail);
  return hipGetLastError();
}

}  // namespace tt
