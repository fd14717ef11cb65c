// Band gather and band embedding in one kernel (fp16 / bf16):
//
//   u_i = gather of band i's (bin, channel) pairs of the complex spectrum (re, im per pair)
//   x0_i = RMSNorm(u_i) W_i^T + b_i            for every band i and frame
//
// ([P1] "The forward chain" and "Band split": each band's bins, stereo-minor inside a bin, re / im
// folded into the feature axis, RMSNorm over the band's features, then a Linear to the model width;
// [P5] export-roformer.py class BandSplit.)  The norm's gain times sqrt(width) is folded into W_i at
// create, so the band norm here is u / max(|u|, 1e-12).
//
// Workgroup = (64 rows (batch, frame) of one band), four waves (two workgroups per compute unit):
//   * gather: thread (row, pair group) reads its pairs for one row straight from the spectrum
//     (for one pair, the 64 rows are 512 contiguous bytes of the [B][F*S][T][2] layout); the row's
//     sum of squares is added up over the pair groups through LDS, and the pairs go into an LDS tile
//     [64 rows][kpad] normalised and in 16 bits, the K padding zero.  The gathered band never goes to
//     HBM;
//   * product: wave w computes features D/4 w .. for the 64 rows on v_mfma_f32_32x32x16 (C^T =
//     W_i u^T: the W_i tiles are the A operand, read from a stream laid out at create in fragment
//     order, 1 KB contiguous per fragment and L2-resident; the tile rows are the B operand, one
//     16-byte LDS read per lane); W fragments are requested two K-step pairs ahead;
//   * epilogue: the products are staged through LDS 32 rows at a time, so x0 + b goes out in whole
//     256-byte row blocks, in fp32 (X) and in 16 bits (XH), with each block's row sum of squares (the
//     row statistic the next consumer turns into the attention norm).
// Bands are walked longest first (a table sorted at create), so the ragged K evens out over the
// device.
#include <algorithm>

#include "kcommon.h"
#include "kernels.h"

namespace mbr {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void mma32(f32x16& c, const f16x8& a, const f16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename T> struct Two;
template <> struct Two<f16> { typedef f16 type __attribute__((ext_vector_type(2))); };
template <> struct Two<bf16> { typedef bf16 type __attribute__((ext_vector_type(2))); };

constexpr int kRows = 64;   // rows (batch, frame) of a band per workgroup
constexpr int kWaves = 4;   // one per SIMD: two workgroups per compute unit fill every SIMD evenly

// FT: 32-feature tiles per wave (D = 128 FT)
template <typename T, int FT, int MAXJ, int LAYOUT>
__global__ __launch_bounds__(64 * kWaves, 2) void embed_kernel(EmbedLaunch L) {
  typedef typename Frag<T>::type frag;
  typedef typename Two<T>::type two;
  constexpr int TH = 64 * kWaves, D = 32 * FT * kWaves, FPW = 32 * FT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* tile = (T*)smem;                          // [kRows][kpad + 8], then the output staging
  __shared__ float part[kWaves][kRows];
  __shared__ float scl[kRows];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int band = L.order[blockIdx.y];
  const int T_ = L.frames, BT = L.batch * T_;
  const int r0 = blockIdx.x * kRows;
  const int foff = L.band_info[4 * band + 0], width = L.band_info[4 * band + 1];
  const int kpad = L.band_info[4 * band + 2];
  const int np = width >> 1, kp2 = kpad >> 1;
  const int stride = kpad + 8;                 // 16-byte row shift: a fragment read is conflict-free

  // ---- gather and normalise (thread = row lane, pair group w: pairs w, w + 4, ...)
  {
    const int row = r0 + lane;
    const int rl = row < BT ? row : BT - 1;    // rows past the end read the last row, never stored
    const int b = rl / T_, t = rl - b * T_;
    const int F = L.n_freqs, S = L.channels;
    const int32_t* pidx = L.gather_pair + (foff >> 1);
    // the pair indices first (wave-uniform: scalar loads, one wait), then every load of the spectrum
    // before any use
    const int wu = __builtin_amdgcn_readfirstlane(w);
    int pj[MAXJ];
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int j = wu + kWaves * u;
      pj[u] = pidx[j < np ? j : np - 1];
    }
    float re[MAXJ], im[MAXJ];
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      re[u] = 0.f;
      im[u] = 0.f;
      if (wu + kWaves * u < np) {              // uniform over the wave
        if constexpr (LAYOUT == 0) {
          const float2 z = *(const float2*)(L.in + (((size_t)b * F * S + pj[u]) * T_ + t) * 2);
          re[u] = z.x;
          im[u] = z.y;
        } else {
          const int f = pj[u] / S, s = pj[u] - f * S;
          const float* base = L.in + ((size_t)b * S * 2 + s * 2) * (size_t)F * T_ + (size_t)f * T_ + t;
          re[u] = base[0];
          im[u] = base[(size_t)F * T_];
        }
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) ss = fmaf(re[u], re[u], fmaf(im[u], im[u], ss));
    part[w][lane] = ss;
    __syncthreads();
    if (tid < kRows) {
      float tot = 0.f;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) tot += part[q][tid];
      scl[tid] = 1.0f / fmaxf(sqrtf(tot), kNormEps);
    }
    __syncthreads();
    const float sc = scl[lane];
    T* trow = tile + lane * stride;
#pragma unroll
    for (int u = 0; u < MAXJ; ++u) {
      const int j = wu + kWaves * u;
      if (j < np) *(two*)(trow + 2 * j) = two{cvt<T>(re[u] * sc), cvt<T>(im[u] * sc)};
    }
    const int padp = kp2 - np;                 // zero pairs of the K padding
    for (int i = tid; i < kRows * padp; i += TH) {
      const int r = i / padp, j = np + (i - r * padp);
      *(two*)(tile + r * stride + 2 * j) = two{cvt<T>(0.f), cvt<T>(0.f)};
    }
    __syncthreads();
  }

  // ---- C^T = W_i u^T: acc[ft][tt] holds features FPW w + 32 ft + (rows of the 32 x 32 tile) for
  // the tile rows 32 tt + lane % 32
  f32x16 acc[FT][2];
#pragma unroll
  for (int i = 0; i < FT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int nks = kpad >> 4;                   // K steps of 16 (even: kpad is a multiple of 32)
  const frag* wf = (const frag*)((const T*)L.W + L.w_off[band]) + (size_t)w * nks * FT * 64 + lane;
  const T* tb0 = tile + (lane & 31) * stride + 8 * (lane >> 5);
  const T* tb1 = tb0 + 32 * stride;
  // K-step pair p: fragments (2p, tile ft) at 2 FT p + ft and (2p + 1, tile ft) at 2 FT p + FT + ft
  auto load = [&](frag (&a)[2 * FT], int p) {
#pragma unroll
    for (int i = 0; i < 2 * FT; ++i) a[i] = wf[(size_t)(2 * FT * p + i) * 64];
  };
  auto step = [&](const frag (&a)[2 * FT], int p) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = 16 * (2 * p + s);
      const frag b0 = *(const frag*)(tb0 + k), b1 = *(const frag*)(tb1 + k);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        mma32(acc[ft][0], a[FT * s + ft], b0);
        mma32(acc[ft][1], a[FT * s + ft], b1);
      }
    }
  };
  // three buffers: the fragments of K-step pair p + 2 are requested while pair p is multiplied
  const int npair = nks >> 1;
  frag A0[2 * FT], A1[2 * FT], A2[2 * FT];
  load(A0, 0);
  if (1 < npair) load(A1, 1);
  for (int p = 0; p < npair; p += 3) {
    if (p + 2 < npair) load(A2, p + 2);
    step(A0, p);
    if (p + 3 < npair) load(A0, p + 3);
    if (p + 1 < npair) step(A1, p + 1);
    if (p + 4 < npair) load(A1, p + 4);
    if (p + 2 < npair) step(A2, p + 2);
  }

  // ---- x0 + b -> X (fp32) and XH (16 bits), and the row sums of squares of each 64-column block:
  // 32 rows at a time staged through LDS (the tile is no longer needed), so that every store writes
  // whole 256-byte row blocks (lane l holds a row's features in fours, scattered over 32 rows)
  constexpr int SR = D + 4;                    // floats per staged row: consecutive rows 16 bytes apart
  constexpr int NBLK = D / 64;
  float* st = (float*)smem;
  const float* bias = L.bias + (size_t)band * D;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    __syncthreads();                           // the tile's last reads / the previous rows' reads
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = acc[ft][tt][4 * q + e];
        *(f32x4*)(st + (lane & 31) * SR + FPW * w + 32 * ft + 8 * q + 4 * (lane >> 5)) = val;
      }
    __syncthreads();
    // 16 lanes per (row, 64-column block), four of them per wave and instruction
    const int g = lane >> 4, c4 = (lane & 15) * 4;
    for (int i = w * 4 + g; i < 32 * NBLK; i += 4 * kWaves) {
      const int rr = i / NBLK, blk = i - rr * NBLK, row = r0 + 32 * tt + rr;
      const int col = 64 * blk + c4;
      const f32x4 a4 = *(const f32x4*)(st + rr * SR + col);
      const f32x4 b4 = *(const f32x4*)(bias + col);
      f32x4 val;
      float q1 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[e] = a4[e] + b4[e];
        q1 = fmaf(val[e], val[e], q1);
      }
      q1 += __shfl_xor(q1, 8, 64);
      q1 += __shfl_xor(q1, 4, 64);
      q1 += __shfl_xor(q1, 2, 64);
      q1 += __shfl_xor(q1, 1, 64);
      if (row < BT) {                          // uniform over the 16 lanes of a row
        const int64_t token = (int64_t)band * BT + row;
        *(f32x4*)(L.X + token * D + col) = val;
        typename Vec4<T>::type h4;
#pragma unroll
        for (int e = 0; e < 4; ++e) h4[e] = cvt<T>(val[e]);
        *(typename Vec4<T>::type*)((T*)L.XH + token * D + col) = h4;
        if ((lane & 15) == 0) L.ss[token * kSsStride + blk] = q1;
      }
    }
  }
}

template <typename T, int FT, int MAXJ>
hipError_t launch_t(const EmbedLaunch& L, hipStream_t stream) {
  constexpr int D = 128 * FT;
  const size_t lds = std::max((size_t)kRows * (L.max_kpad + 8) * sizeof(T), (size_t)32 * (D + 4) * 4);
  const int BT = L.batch * L.frames;
  const dim3 grid((unsigned)((BT + kRows - 1) / kRows), (unsigned)L.num_bands), block(64 * kWaves);
  const void* k = L.layout == 0 ? (const void*)embed_kernel<T, FT, MAXJ, 0> : (const void*)embed_kernel<T, FT, MAXJ, 1>;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (L.layout == 0) hipLaunchKernelGGL((embed_kernel<T, FT, MAXJ, 0>), grid, block, lds, stream, L);
  else hipLaunchKernelGGL((embed_kernel<T, FT, MAXJ, 1>), grid, block, lds, stream, L);
  return hipGetLastError();
}

// pairs per thread: the widest band's pairs over the four pair groups (272 pairs at most: kpad 544)
template <typename T, int FT>
hipError_t launch_w(const EmbedLaunch& L, hipStream_t stream) {
  const int per = (L.max_kpad / 2 + kWaves - 1) / kWaves;
  if (per <= 24) return launch_t<T, FT, 24>(L, stream);
  if (per <= 68) return launch_t<T, FT, 68>(L, stream);
  return hipErrorInvalidValue;
}

}  // namespace

bool embed_fused_supported(int dtype, int D, int max_kpad) {
  return dtype != DT_F32 && (D == 384 || D == 512) && max_kpad <= 544;
}

hipError_t launch_embed(const EmbedLaunch& L, hipStream_t stream) {
  if (!embed_fused_supported(L.dtype, L.D, L.max_kpad) || L.batch < 1 || L.frames < 1) return hipErrorInvalidValue;
  if (L.dtype == DT_F16) return L.D == 384 ? launch_w<f16, 3>(L, stream) : launch_w<f16, 4>(L, stream);
  return L.D == 384 ? launch_w<bf16, 3>(L, stream) : launch_w<bf16, 4>(L, stream);
}

}  // namespace mbr
