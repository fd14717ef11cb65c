// Memory-bound passes of the core: row norms of the residual stream, the band gather with its
// per-band normalisation, and the inverse-index mask average.
#include "kcommon.h"
#include "kernels.h"

namespace mbr {

namespace {

// ---------------------------------------------------------------------------------- row norm
// RMSNorm of the pages ([P1] the RMSNorm paragraph under BandSplit): x / max(||x||, 1e-12) times
// sqrt(d) times gamma.  One wave per row; lane l holds elements l, l+64, ...  The gains of the
// norms that feed a projection are folded into that projection's weights, so the pre-projection
// output here is x * sqrt(D) / max(||x||, eps); the Transformer's output norm applies its gain.
// Gates of the attention ([P1] "Per Attention layer": to_gates on the normalised input, sigmoid,
// one per head) are computed from the same fp32 normalised row.
template <typename T, int NPL>
__global__ __launch_bounds__(256) void norm_kernel(NormLaunch L) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= L.rows) return;
  const int D = L.D;
  float* x = L.x + (size_t)row * D;
  float v[NPL];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    v[j] = x[lane + 64 * j];
    ss += v[j] * v[j];
  }
  ss = wave_sum(ss);
  const float sqrtD = sqrtf((float)D);
  if (L.mode != 0) {
    const float inv = 1.0f / fmaxf(sqrtf(ss), kNormEps);
    ss = 0.f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      v[j] = v[j] * inv * L.gain[lane + 64 * j];
      x[lane + 64 * j] = v[j];
      ss += v[j] * v[j];
    }
    ss = wave_sum(ss);
  }
  T* xh = (T*)L.xh + (size_t)row * D;
  if (L.mode == 2) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) xh[lane + 64 * j] = cvt<T>(v[j]);
    return;
  }
  const float k = sqrtD / fmaxf(sqrtf(ss), kNormEps);
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    v[j] *= k;
    xh[lane + 64 * j] = cvt<T>(v[j]);
  }
  if (L.gates) {
    for (int h = 0; h < L.H; ++h) {
      const float* w = L.wg + (size_t)h * D;
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) a += v[j] * w[lane + 64 * j];
      a = wave_sum(a);
      if (lane == 0) L.gates[(size_t)row * L.H + h] = sigmoidf_(a + L.bg[h]);
    }
  }
}

// The same passes for D a multiple of 128: 32 lanes per row (two rows per wave), 16-byte loads
// and stores, reductions over the 32 lanes of the row.
template <typename T, int NV>
__global__ __launch_bounds__(256) void norm4_kernel(NormLaunch L) {
  typedef typename Vec4<T>::type h4;
  const int lane = threadIdx.x & 63, l = lane & 31;
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const bool valid = row < L.rows;
  const int D = L.D, D4 = D >> 2;
  float4* x4 = (float4*)L.x + (size_t)(valid ? row : 0) * D4;
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    v[j] = valid ? x4[l + 32 * j] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float sqrtD = sqrtf((float)D);
  if (L.mode != 0) {
    const float inv = 1.0f / fmaxf(sqrtf(ss), kNormEps);
    const float4* g4 = (const float4*)L.gain;
    ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const float4 gg = g4[l + 32 * j];
      v[j] = make_float4(v[j].x * inv * gg.x, v[j].y * inv * gg.y, v[j].z * inv * gg.z, v[j].w * inv * gg.w);
      if (valid) x4[l + 32 * j] = v[j];
      ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  }
  h4* xh = (h4*)((T*)L.xh + (size_t)(valid ? row : 0) * D);
  const float k = L.mode == 2 ? 1.0f : sqrtD / fmaxf(sqrtf(ss), kNormEps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    v[j] = make_float4(v[j].x * k, v[j].y * k, v[j].z * k, v[j].w * k);
    h4 o;
    o[0] = cvt<T>(v[j].x); o[1] = cvt<T>(v[j].y); o[2] = cvt<T>(v[j].z); o[3] = cvt<T>(v[j].w);
    if (valid) xh[l + 32 * j] = o;
  }
  if (L.mode != 2 && L.gates) {
    for (int h = 0; h < L.H; ++h) {
      const float4* w4 = (const float4*)(L.wg + (size_t)h * D);
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const float4 ww = w4[l + 32 * j];
        a += v[j].x * ww.x + v[j].y * ww.y + v[j].z * ww.z + v[j].w * ww.w;
      }
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
      if (valid && l == 0) L.gates[(size_t)row * L.H + h] = sigmoidf_(a + L.bg[h]);
    }
  }
}

template <typename T>
hipError_t norm_t(const NormLaunch& L, hipStream_t stream) {
  if (L.D % 128 == 0) {
    dim3 grid((L.rows + 7) / 8), block(256);
    switch (L.D / 128) {
      case 1: hipLaunchKernelGGL((norm4_kernel<T, 1>), grid, block, 0, stream, L); break;
      case 2: hipLaunchKernelGGL((norm4_kernel<T, 2>), grid, block, 0, stream, L); break;
      case 3: hipLaunchKernelGGL((norm4_kernel<T, 3>), grid, block, 0, stream, L); break;
      case 4: hipLaunchKernelGGL((norm4_kernel<T, 4>), grid, block, 0, stream, L); break;
      case 5: hipLaunchKernelGGL((norm4_kernel<T, 5>), grid, block, 0, stream, L); break;
      case 6: hipLaunchKernelGGL((norm4_kernel<T, 6>), grid, block, 0, stream, L); break;
      case 7: hipLaunchKernelGGL((norm4_kernel<T, 7>), grid, block, 0, stream, L); break;
      case 8: hipLaunchKernelGGL((norm4_kernel<T, 8>), grid, block, 0, stream, L); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid((L.rows + 3) / 4), block(256);
  switch (L.D / 64) {
    case 1: hipLaunchKernelGGL((norm_kernel<T, 1>), grid, block, 0, stream, L); break;
    case 2: hipLaunchKernelGGL((norm_kernel<T, 2>), grid, block, 0, stream, L); break;
    case 3: hipLaunchKernelGGL((norm_kernel<T, 3>), grid, block, 0, stream, L); break;
    case 4: hipLaunchKernelGGL((norm_kernel<T, 4>), grid, block, 0, stream, L); break;
    case 5: hipLaunchKernelGGL((norm_kernel<T, 5>), grid, block, 0, stream, L); break;
    case 6: hipLaunchKernelGGL((norm_kernel<T, 6>), grid, block, 0, stream, L); break;
    case 7: hipLaunchKernelGGL((norm_kernel<T, 7>), grid, block, 0, stream, L); break;
    case 8: hipLaunchKernelGGL((norm_kernel<T, 8>), grid, block, 0, stream, L); break;
    case 9: hipLaunchKernelGGL((norm_kernel<T, 9>), grid, block, 0, stream, L); break;
    case 10: hipLaunchKernelGGL((norm_kernel<T, 10>), grid, block, 0, stream, L); break;
    case 11: hipLaunchKernelGGL((norm_kernel<T, 11>), grid, block, 0, stream, L); break;
    case 12: hipLaunchKernelGGL((norm_kernel<T, 12>), grid, block, 0, stream, L); break;
    case 13: hipLaunchKernelGGL((norm_kernel<T, 13>), grid, block, 0, stream, L); break;
    case 14: hipLaunchKernelGGL((norm_kernel<T, 14>), grid, block, 0, stream, L); break;
    case 15: hipLaunchKernelGGL((norm_kernel<T, 15>), grid, block, 0, stream, L); break;
    case 16: hipLaunchKernelGGL((norm_kernel<T, 16>), grid, block, 0, stream, L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------- band gather
// One (re, im) pair of the output in one LDS / global unit: 4 bytes for 16-bit types, 8 for fp32.
template <typename T> struct PairUnit;
template <> struct PairUnit<float> { typedef float2 type; static __device__ type make(float a, float b) { return make_float2(a, b); } };
template <> struct PairUnit<f16> {
  typedef uint32_t type;
  static __device__ type make(float a, float b) {
    const f16 x = cvt<f16>(a), y = cvt<f16>(b);
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  }
};
template <> struct PairUnit<bf16> {
  typedef uint32_t type;
  static __device__ type make(float a, float b) {
    const bf16 x = cvt<bf16>(a), y = cvt<bf16>(b);
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  }
};

// Band gather with the band's RMSNorm ([P1] "The forward chain", BandSplit): for 64 frames of one
// band, each lane (one frame) reads the band's (re, im) pairs along its frames (coalesced along
// the time axis of the input), the row norm comes from a first pass, and the normalised pairs are
// transposed through LDS (rows of kpad/2 + 1 units, so the 64 lanes of a column write fall on
// distinct banks) into the band's block of U, whose rows (frames) are contiguous.
template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void gather_kernel(GatherLaunch L) {
  typedef typename PairUnit<T>::type P;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  P* tile = (P*)lds_raw;                       // [64][kpad/2 + 1]
  int* pidx = (int*)(tile + 64 * (L.max_kpad / 2 + 1));   // the band's pair indices
  __shared__ float part[4][64];
  __shared__ float scale[64];
  const int band = blockIdx.z, b = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const int lane = threadIdx.x & 63, wq = threadIdx.x >> 6;
  const int t = t0 + lane;
  const bool valid = t < L.frames;
  const int foff = L.band_info[band * 4 + 0], width = L.band_info[band * 4 + 1];
  const int kpad = L.band_info[band * 4 + 2], ucol = L.band_info[band * 4 + 3];
  const int npairs = width / 2, kp2 = kpad / 2, rs = kp2 + 1;
  const int F = L.n_freqs, S = L.channels, FS = F * S, T_ = L.frames;
  for (int j = threadIdx.x; j < npairs; j += 256) pidx[j] = L.gather_pair[foff / 2 + j];
  __syncthreads();
  // lanes past the last frame read frame T-1 and are never stored
  const int tl = valid ? t : T_ - 1;
  auto load = [&](int p, float& re, float& im) {
    if constexpr (LAYOUT == 0) {
      const float2 z = *(const float2*)(L.in + (((size_t)b * FS + p) * T_ + tl) * 2);
      re = z.x; im = z.y;
    } else {
      const int f = p / S, s = p - f * S;
      const float* base = L.in + ((size_t)b * S * 2 + s * 2) * (size_t)F * T_ + (size_t)f * T_ + tl;
      re = base[0];
      im = base[(size_t)F * T_];
    }
  };
  float ss = 0.f;
#pragma unroll 16
  for (int j = wq; j < npairs; j += 4) {
    float re, im;
    load(pidx[j], re, im);
    ss += re * re + im * im;
  }
  part[wq][lane] = ss;
  __syncthreads();
  if (wq == 0) {
    const float tot = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    scale[lane] = 1.0f / fmaxf(sqrtf(tot), kNormEps);
  }
  __syncthreads();
  const float sc = scale[lane];
  // sixteen pairs per batch: all index reads, then all loads, then all LDS stores (the stores would
  // otherwise keep the next index read, and so the next load, waiting)
  for (int j0 = wq; j0 < npairs; j0 += 64) {
    float re[16], im[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = j0 + 4 * u;
      const int pj = pidx[j < npairs ? j : j0];
      load(pj, re[u], im[u]);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = j0 + 4 * u;
      if (j < npairs) tile[lane * rs + j] = PairUnit<T>::make(re[u] * sc, im[u] * sc);
    }
  }
  for (int j = npairs + wq; j < kp2; j += 4) tile[lane * rs + j] = PairUnit<T>::make(0.f, 0.f);
  __syncthreads();
  // rows b*T + t0 .. of band `band`: contiguous in U at column block ucol, kpad/2 units a row
  const int rows = min(64, T_ - t0);
  const size_t BT = (size_t)L.batch * T_;
  P* dst = (P*)((T*)L.U + (size_t)ucol * BT + ((size_t)b * T_ + t0) * kpad);
  for (int r = wq; r < rows; r += 4)
    for (int c = lane; c < kp2; c += 64) dst[(size_t)r * kp2 + c] = tile[r * rs + c];
}

// The same gather for bands of up to 16 * MAXJ pairs, with more workgroups and one read of the
// input: 16 frames of one band per workgroup; lane l of wave w takes frame t0 + l % 16 and the
// band's pairs g, g + 16, ... (g = 4w + l / 16), holds them in registers while the band norm is
// summed (through LDS) and writes them normalised into an LDS tile (rows of kpad/2 + 1 units) that
// goes out as the band's 16 contiguous rows of U.  For one pair, 16 frames are 128 contiguous bytes
// of the input.
template <typename T, int LAYOUT, int MAXJ>
__global__ __launch_bounds__(256) void gather16_kernel(GatherLaunch L) {
  typedef typename PairUnit<T>::type P;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  P* tile = (P*)lds_raw;                       // [16][kpad/2 + 1]
  __shared__ float part[16][17];               // [pair group][frame]
  __shared__ float scale[16];
  const int band = blockIdx.z, b = blockIdx.y;
  const int t0 = blockIdx.x * 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int fr = lane & 15, g = 4 * w + (lane >> 4);
  const int T_ = L.frames;
  const int t = t0 + fr;
  const int tl = t < T_ ? t : T_ - 1;          // frames past the end read the last one, never stored
  const int foff = L.band_info[band * 4 + 0], width = L.band_info[band * 4 + 1];
  const int kpad = L.band_info[band * 4 + 2], ucol = L.band_info[band * 4 + 3];
  const int npairs = width / 2, kp2 = kpad / 2, rs = kp2 + 1;
  const int F = L.n_freqs, S = L.channels, FS = F * S;
  const int32_t* pidx = L.gather_pair + foff / 2;
  int pj[MAXJ];
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) {
    const int j = g + 16 * u;
    pj[u] = pidx[j < npairs ? j : 0];
  }
  float re[MAXJ], im[MAXJ];
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) {
    if constexpr (LAYOUT == 0) {
      const float2 z = *(const float2*)(L.in + (((size_t)b * FS + pj[u]) * T_ + tl) * 2);
      re[u] = z.x;
      im[u] = z.y;
    } else {
      const int f = pj[u] / S, s = pj[u] - f * S;
      const float* base = L.in + ((size_t)b * S * 2 + s * 2) * (size_t)F * T_ + (size_t)f * T_ + tl;
      re[u] = base[0];
      im[u] = base[(size_t)F * T_];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < MAXJ; ++u)
    if (g + 16 * u < npairs) ss += re[u] * re[u] + im[u] * im[u];
  part[g][fr] = ss;
  __syncthreads();
  if (threadIdx.x < 16) {
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) tot += part[q][threadIdx.x];
    scale[threadIdx.x] = 1.0f / fmaxf(sqrtf(tot), kNormEps);
  }
  __syncthreads();
  const float sc = scale[fr];
#pragma unroll
  for (int u = 0; u < MAXJ; ++u) {
    const int j = g + 16 * u;
    if (j < npairs) tile[fr * rs + j] = PairUnit<T>::make(re[u] * sc, im[u] * sc);
  }
  for (int i = threadIdx.x; i < 16 * (kp2 - npairs); i += 256) {
    const int r = i / (kp2 - npairs), j = npairs + i - r * (kp2 - npairs);
    tile[r * rs + j] = PairUnit<T>::make(0.f, 0.f);
  }
  __syncthreads();
  // rows b*T + t0 .. of band `band`: contiguous in U at column block ucol, kpad/2 units a row
  const int rows = min(16, T_ - t0);
  const size_t BT = (size_t)L.batch * T_;
  P* dst = (P*)((T*)L.U + (size_t)ucol * BT + ((size_t)b * T_ + t0) * kpad);
  for (int r = w; r < rows; r += 4)
    for (int c = lane; c < kp2; c += 64) dst[(size_t)r * kp2 + c] = tile[r * rs + c];
}

// ---------------------------------------------------------------------------------- average
// [P1] "The forward chain": the band masks go back to their (bin, channel) pairs and each value
// is divided by the number of bands covering its bin.  Instead of a scatter with atomics, every
// output element reads its (at most two) sources through the inverse index and multiplies by the
// precomputed 1/count: deterministic, one write per element.  Threads run along frames.
__global__ __launch_bounds__(256) void average_kernel(AverageLaunch L) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int p = blockIdx.y;                   // pair f*S + s
  const int bs = blockIdx.z;                  // b * stems + stem
  if (t >= L.frames) return;
  const int T_ = L.frames, S = L.channels, F = L.n_freqs;
  const int b = bs / L.stems, st = bs - b * L.stems;
  const int s1 = L.inv_slot[2 * p], s2 = L.inv_slot[2 * p + 1];
  const float w = L.inv_weight[p];
  const float* M = L.M + ((size_t)st * L.batch + b) * (size_t)L.total * T_;
  float re = M[(size_t)(2 * s1) * T_ + t], im = M[(size_t)(2 * s1 + 1) * T_ + t];
  if (s2 >= 0) {
    re += M[(size_t)(2 * s2) * T_ + t];
    im += M[(size_t)(2 * s2 + 1) * T_ + t];
  }
  re *= w;
  im *= w;
  if (L.layout == 0) {
    *(float2*)(L.out + (((size_t)bs * F * S + p) * T_ + t) * 2) = make_float2(re, im);
  } else {
    const int f = p / S, s = p - f * S;
    float* base = L.out + ((size_t)bs * S * 2 + s * 2) * (size_t)F * T_ + (size_t)f * T_ + t;
    base[0] = re;
    base[(size_t)F * T_] = im;
  }
}

// The same with four consecutive frames per thread (16-byte reads of the masks, 32 contiguous bytes
// written per thread in the (pair, frame, re / im) layout) and one wave per workgroup, when the
// frame count is a multiple of 4: a quarter of the threads and memory instructions.
__global__ __launch_bounds__(64) void average4_kernel(AverageLaunch L) {
  const int t = (blockIdx.x * 64 + threadIdx.x) * 4;
  const int p = blockIdx.y;                   // pair f*S + s
  const int bs = blockIdx.z;                  // b * stems + stem
  if (t >= L.frames) return;
  const int T_ = L.frames, S = L.channels, F = L.n_freqs;
  const int b = bs / L.stems, st = bs - b * L.stems;
  const int s1 = L.inv_slot[2 * p], s2 = L.inv_slot[2 * p + 1];
  const float w = L.inv_weight[p];
  const float* M = L.M + ((size_t)st * L.batch + b) * (size_t)L.total * T_;
  f32x4 re = *(const f32x4*)(M + (size_t)(2 * s1) * T_ + t), im = *(const f32x4*)(M + (size_t)(2 * s1 + 1) * T_ + t);
  if (s2 >= 0) {
    re += *(const f32x4*)(M + (size_t)(2 * s2) * T_ + t);
    im += *(const f32x4*)(M + (size_t)(2 * s2 + 1) * T_ + t);
  }
  re *= w;
  im *= w;
  if (L.layout == 0) {
    f32x4* o = (f32x4*)(L.out + (((size_t)bs * F * S + p) * T_ + t) * 2);
    o[0] = f32x4{re[0], im[0], re[1], im[1]};
    o[1] = f32x4{re[2], im[2], re[3], im[3]};
  } else {
    const int f = p / S, s = p - f * S;
    float* base = L.out + ((size_t)bs * S * 2 + s * 2) * (size_t)F * T_ + (size_t)f * T_ + t;
    *(f32x4*)base = re;
    *(f32x4*)(base + (size_t)F * T_) = im;
  }
}

__global__ __launch_bounds__(256) void gelu_kernel(const float* x, float* y, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = gelu_erf(x[i]);
}

}  // namespace

hipError_t launch_gelu(const float* x, float* y, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gelu_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

hipError_t launch_norm(const NormLaunch& L, hipStream_t stream) {
  if (L.rows <= 0) return hipSuccess;
  if (L.D % 64 || L.D > 1024) return hipErrorInvalidValue;
  switch (L.dtype) {
    case DT_F32: return norm_t<float>(L, stream);
    case DT_F16: return norm_t<f16>(L, stream);
    case DT_BF16: return norm_t<bf16>(L, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int LAYOUT, int MAXJ>
hipError_t gather16_t(const GatherLaunch& L, hipStream_t stream) {
  dim3 grid((L.frames + 15) / 16, L.batch, L.num_bands), block(256);
  const size_t lds = (size_t)16 * (L.max_kpad / 2 + 1) * 2 * sizeof(T);
  hipError_t e = hipFuncSetAttribute((const void*)gather16_kernel<T, LAYOUT, MAXJ>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gather16_kernel<T, LAYOUT, MAXJ>), grid, block, lds, stream, L);
  return hipGetLastError();
}

template <typename T>
hipError_t gather_t(const GatherLaunch& L, hipStream_t stream) {
  // bands of up to 384 pairs: 16 frames per workgroup, pairs held in registers
  const int maxp = L.max_kpad / 2;
  if (maxp <= 16 * 8) return L.layout == 0 ? gather16_t<T, 0, 8>(L, stream) : gather16_t<T, 1, 8>(L, stream);
  if (maxp <= 16 * 24) return L.layout == 0 ? gather16_t<T, 0, 24>(L, stream) : gather16_t<T, 1, 24>(L, stream);
  dim3 grid((L.frames + 63) / 64, L.batch, L.num_bands), block(256);
  const size_t lds = (size_t)64 * (L.max_kpad / 2 + 1) * 2 * sizeof(T) + (size_t)(L.max_kpad / 2) * 4;
  if (lds > 160 * 1024 - 2048) return hipErrorInvalidValue;
  const void* k = L.layout == 0 ? (const void*)gather_kernel<T, 0> : (const void*)gather_kernel<T, 1>;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (L.layout == 0) hipLaunchKernelGGL((gather_kernel<T, 0>), grid, block, lds, stream, L);
  else hipLaunchKernelGGL((gather_kernel<T, 1>), grid, block, lds, stream, L);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherLaunch& L, hipStream_t stream) {
  switch (L.dtype) {
    case DT_F32: return gather_t<float>(L, stream);
    case DT_F16: return gather_t<f16>(L, stream);
    case DT_BF16: return gather_t<bf16>(L, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_average(const AverageLaunch& L, hipStream_t stream) {
  if (L.frames % 4 == 0) {   // rows of the masks and of the output then start 16-byte aligned
    dim3 grid((L.frames / 4 + 63) / 64, L.n_freqs * L.channels, L.batch * L.stems), block(64);
    hipLaunchKernelGGL(average4_kernel, grid, block, 0, stream, L);
    return hipGetLastError();
  }
  dim3 grid((L.frames + 255) / 256, L.n_freqs * L.channels, L.batch * L.stems), block(256);
  hipLaunchKernelGGL(average_kernel, grid, block, 0, stream, L);
  return hipGetLastError();
}

}  // namespace mbr
