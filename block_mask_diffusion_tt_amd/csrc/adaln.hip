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

// u = SiLU(emb) W (+ bias) on the matrix cores (v_mfma_f32_32x32x16_bf16).
// W is bf16; each fp32 value x of SiLU(emb) is split exactly into three
// bf16 parts, x = hi + mid + lo (hi the top 8 significant bits of x, mid the
// top 8 of x - hi, lo the at most 8 bits left), so every product of the
// three bf16 matrix products is exact and only the fp32 accumulation rounds,
// as in a fp32 dot product.
//   Workgroup = 8 waves over a tile of 32 sequences x 128 columns: wave
// (nt, kh) multiplies the 32 columns of n-tile nt over the 128 values of k in
// half kh, and the two halves are summed through LDS in a fixed order.  Every
// workgroup computes SiLU for its rows itself, so the tile is wide in
// columns (fewer workgroups repeat that work).  The 512 threads copy the
// tile's W slab (256 x 128 bf16) into LDS and compute the split SiLU values
// of its 32 rows into LDS once; the B operands (W, column per lane) come out
// of the slab through the transposing ds_read_b64_tr_b16.  The time goes to
// fetching the W slab and writing the n_layers copies, not to arithmetic, so
// every load of the kernel is issued before its first wait.
// The epilogue adds the bias and writes every layer's copy with its table
// row: wave (nt, kh) writes the layers l with l % 2 == kh, 32 consecutive
// columns (128 bytes) per row and store.
//   Operand layout: lane l holds row (A) or column (B) l % 32 and 8 values of
// k; element e of lane l is k = 16 m + 4 (l / 32) + (e % 4) + 8 (e / 4) for
// k-step m, on both sides.  The accumulator holds column l % 32 and rows
// 8 (r / 4) + 4 (l / 32) + r % 4, r = 0..15.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileB = 32;                // sequences per workgroup
constexpr int kTileN = 128;               // columns per workgroup (4 n-tiles)
constexpr int kSplits = 3;                // bf16 parts of each SiLU value
constexpr int kEPitch = kEmb + 8;         // bf16 per LDS row of a part (16 bytes of
                                          // padding spread 16 rows over all banks)
constexpr int kKSteps = kEmb / 16 / 2;    // k-steps per wave (one half of k)
constexpr int kPreLayers = 8;             // table values loaded up front per lane
                                          // (layers kh, kh + 2, ...: up to 16 layers)

// Position of k within its 16-block in the SiLU rows: groups of 4 in the
// order 0, 2, 1, 3, so that a lane's 8 values are 16 contiguous bytes.
__device__ __forceinline__ int epos(int k) {
  const int g = (k >> 2) & 3;
  return (k & ~15) + 4 * ((g & 1) * 2 + (g >> 1)) + (k & 3);
}

// Byte offset of W slab element (k, c), c < 128: rows of 256 bytes, the
// 64-byte chunk of each n-tile XOR-swizzled with k % 4 so that the 8 rows
// of one transposing read hit all banks.
__device__ __forceinline__ int wpos(int k, int c) {
  return k * (kTileN * 2) + ((((c >> 5) ^ k) & 3) << 6) + (c & 31) * 2;
}

__global__ __launch_bounds__(512) void adaln_kernel(int B, int width, int n_layers,
                                                    const float* __restrict__ emb,
                                                    const uint16_t* __restrict__ w,
                                                    const float* __restrict__ bias,
                                                    const float* __restrict__ table,
                                                    float* __restrict__ ada) {
  __shared__ __attribute__((aligned(16))) uint16_t s_e[kSplits][kTileB][kEPitch];
  __shared__ __attribute__((aligned(16))) uint8_t s_w[kEmb * kTileN * 2];
  __shared__ float s_red[4][2][16][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
  const int nt = wave & 3, kh = wave >> 2;
  const int l32 = lane & 31, half = lane >> 5, grp = lane >> 4, li = lane & 15;
  const int N = 3 * width;
  const int b0 = blockIdx.y * kTileB;
  const int n0 = blockIdx.x * kTileN;

  // All loads are issued up front and without branches (out-of-range rows,
  // columns and layers read a valid element whose value is then replaced by
  // zero or not used),
  // so that the compiler's waits can count them in order: the SiLU work
  // waits for the embedding rows only, while W, the bias and the table rows
  // are still in flight, and the kernel waits for memory once.
  //   The tile's embedding rows: thread t takes row t / 16 and the 4-value
  // groups k = 64 i + 4 (t % 16).
  const int er_row = tid >> 4, er_q = tid & 15;
  const bool rv = b0 + er_row < B;
  float x[kEmb / 64][4];
  {
    const float* er = emb + static_cast<int64_t>(rv ? b0 + er_row : 0) * kEmb + 4 * er_q;
#pragma unroll
    for (int i = 0; i < kEmb / 64; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[i][j] = er[64 * i + j];
  }

  // W slab: 8-byte pieces (4 columns; w is 8-byte aligned and N a multiple
  // of 4), 16 rows per pass
  const int wc = 4 * (tid & 31), wr = tid >> 5;
  const bool cv = n0 + wc < N;
  uint2 wv[kEmb * kTileN / 4 / 512];
  {
    const uint16_t* const wp = w + static_cast<int64_t>(wr) * N + (cv ? n0 + wc : 0);
#pragma unroll
    for (int i = 0; i < kEmb * kTileN / 4 / 512; ++i)
      wv[i] = *reinterpret_cast<const uint2*>(wp + static_cast<int64_t>(16 * i) * N);
  }

  // what the epilogue adds: the bias and the table rows of this wave's
  // layers kh, kh + 2, ... (a missing vector reads emb[0])
  const int n = n0 + 32 * nt + l32;   // this lane's column
  const bool ncol = n < N;
  const int which = ncol ? n / width : 0;   // shift, scale or gate
  const int c = ncol ? n - which * width : 0;
  float bv = (bias ? bias : emb)[bias ? c + which * width : 0];
  float tv[kPreLayers];
#pragma unroll
  for (int p = 0; p < kPreLayers; ++p) {
    const int l = min(kh + 2 * p, n_layers - 1);
    tv[p] = (table ? table : emb)[table ? (static_cast<int64_t>(l) * 3 + which) * width + c : 0];
  }

  // SiLU of the tile's rows, split into three bf16 parts, into LDS
  {
    const int r = er_row, q = er_q;
#pragma unroll
    for (int i = 0; i < kEmb / 64; ++i) {
      uint32_t part[kSplits][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // hardware exp2 and reciprocal: a few ulp, far inside the fp32 sum's error
        const float v = rv ? x[i][j] : 0.f;
        const float s = v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(v * -1.44269504f));
        const uint32_t h = __float_as_uint(s) & 0xffff0000u;
        const float r1 = s - __uint_as_float(h);
        const uint32_t m = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(m);   // at most 8 significant bits
        part[0][j] = h;
        part[1][j] = m;
        part[2][j] = __float_as_uint(r2);
      }
      const int pos = epos(64 * i + 4 * q);
#pragma unroll
      for (int sp = 0; sp < kSplits; ++sp) {
        const u32x2 pk = {__builtin_amdgcn_perm(part[sp][1], part[sp][0], 0x07060302u),
                          __builtin_amdgcn_perm(part[sp][3], part[sp][2], 0x07060302u)};
        *reinterpret_cast<u32x2*>(&s_e[sp][r][pos]) = pk;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kEmb * kTileN / 4 / 512; ++i) {
    const u32x2 v = {cv ? wv[i].x : 0u, cv ? wv[i].y : 0u};
    *reinterpret_cast<u32x2*>(&s_w[wpos(wr + 16 * i, wc)]) = v;
  }
  __syncthreads();

  // three accumulators (one per part): independent chains of 8 products
  f32x16 acc[kSplits];
#pragma unroll
  for (int sp = 0; sp < kSplits; ++sp)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[sp][i] = 0.f;
  // this lane's transposing reads: rows 16 m + 4 half + li / 4 (+ 8), columns
  // 32 nt + 16 (grp & 1) + 4 (li & 3); lane j of each 16-lane group receives
  // column j of the 4 rows
  const int wcol = 32 * nt + 16 * (grp & 1) + 4 * (li & 3);
  typedef __attribute__((address_space(3))) uint8_t LdsU8;
  typedef __attribute__((address_space(3))) v4i16 LdsV4;
  LdsU8* const lw = (LdsU8*)(s_w);   // address-space cast
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    const int m = kh * kKSteps + ks;
    const int k = 16 * m + 4 * half + (li >> 2);
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<LdsV4*>(lw + wpos(k, wcol)));
    const v4i16 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<LdsV4*>(lw + wpos(k + 8, wcol)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 wb = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
    const bf16x8 bop = __builtin_bit_cast(bf16x8, wb);
#pragma unroll
    for (int sp = 0; sp < kSplits; ++sp) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(&s_e[sp][l32][16 * m + 8 * half]);
      acc[sp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bop,
                                                        acc[sp], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) s_red[nt][kh][i][lane] = (acc[2][i] + acc[1][i]) + acc[0][i];
  __syncthreads();
  if (!ncol) return;
  if (!bias) bv = 0.f;
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = (s_red[nt][0][i][lane] + s_red[nt][1][i][lane]) + bv;
  const int nrows = min(kTileB, B - b0) - 4 * half;   // rows left from this lane's first
  float* const base = ada + (static_cast<int64_t>(which) * B + b0 + 4 * half) * width + c;
  const int64_t layer = static_cast<int64_t>(3) * B * width;
  auto store_layer = [&](int l, float t) {
    float* const dst = base + l * layer;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // row offset, the same in every lane (kept scalar: a 32-bit scalar
      // product per row instead of a 64-bit vector one per row and lane)
      const int rb = 8 * (i >> 2) + (i & 3);
      const int off = __builtin_amdgcn_readfirstlane(rb * width);
      if (rb < nrows) dst[off] = u[i] + t;
    }
  };
#pragma unroll
  for (int p = 0; p < kPreLayers; ++p)
    if (kh + 2 * p < n_layers) store_layer(kh + 2 * p, table ? tv[p] : 0.f);
  for (int l = kh + 2 * kPreLayers; l < n_layers; l += 2)
    store_layer(l, table ? table[(static_cast<int64_t>(l) * 3 + which) * width + c] : 0.f);
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
  const dim3 grid(static_cast<unsigned>(ceil_div(N, kTileN)), static_cast<unsigned>(ceil_div(B, kTileB)));
  hipLaunchKernelGGL(adaln_kernel, grid, dim3(512), 0, st, B, width, n_layers, emb,
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
