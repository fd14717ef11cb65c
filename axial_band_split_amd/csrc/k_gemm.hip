// MFMA GEMM family of the core: C = A . B^T with fused epilogues.
//
// The linear layers of the core ([P1] "Per Attention layer", "Parameter accounting"; [P5]
// export-roformer.py classes Attn, FF and the mask MLP) all reduce to this form with the weight
// kept in its [out, in] layout, so both operands stream along K.  One 256-thread workgroup computes
// a BM x BN tile with 2 x 2 waves, each wave a (BM/2) x (BN/2) block of 16 x 16 matrix-core tiles;
// K advances 64 bytes a step through a double-buffered LDS stage.
//
// Epilogues (applied to the fp32 accumulators in registers):
//   EMBED  band embedding: + bias, fp32 residual stream out
//   QKV    rotary on q and k (interleaved pairs, partner column = neighbouring lane), q / k / v
//          scattered into the per-sequence attention layout of the current axis
//   GELU   + bias, exact-erf GELU, operand dtype out
//   RESID  + bias (optional), added into the fp32 residual stream
//   TANH   + bias, tanh, operand dtype out
//   GLU    value and gate columns arrive paired in neighbouring 16-column tiles (the weights are
//          repacked that way); value * sigmoid(gate) is stored feature-major for the average
#include "kcommon.h"
#include "kernels.h"

namespace mbr {

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 80;  // 64 data bytes of a K step + 16 bytes of padding per LDS row

template <typename T, int EPI, int BM, int BN>
struct GemmKernel {
  static constexpr int EPF = Frag<T>::EPF;
  static constexpr int BK = 4 * EPF;          // K elements per step
  static constexpr int TM = BM / 32, TN = BN / 32;
  static constexpr int CHUNKS = (BM + BN) * 4;
  static constexpr int PER = CHUNKS / kThreads;
  static_assert(CHUNKS % kThreads == 0, "tile loader");
  using frag = typename Frag<T>::type;

  __device__ static void epilogue(const GemmLaunch& L, const GemmGroup& g, int M, int rb, int cb,
                                  f32x4 (&acc)[TM][TN], int lane) {
    const int g4 = lane >> 4, l16 = lane & 15;
    if constexpr (EPI == EPI_QKV) {
      const QkvArgs& a = L.qkv;
      const int I = a.heads * a.dh;
      const int BT = a.batch * a.frames;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = cb + j * 16 + l16;
        const int which = col / I;             // 0 q, 1 k, 2 v (uniform over a 16-column tile)
        const int f = col - which * I;
        const int h = f / a.dh, d = f - h * a.dh;
        const bool even = (d & 1) == 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rb + i * 16 + 4 * g4 + r;
            float v = acc[i][j][r];
            const float partner = __shfl_xor(v, 1, 64);
            if (row >= M || col >= g.N) continue;
            int seq, pos;
            if (a.axis == 0) { seq = row / a.frames; pos = row - seq * a.frames; }
            else { pos = row / BT; seq = row - pos * BT; }
            if (which < 2) {
              const int pj = pos * (a.dh >> 1) + (d >> 1);
              const float c = a.cos[pj], s = a.sin[pj];
              v = even ? v * c - partner * s : partner * s + v * c;
              T* dst = (T*)(which == 0 ? a.q : a.k);
              dst[(((size_t)seq * a.heads + h) * a.npad + pos) * a.dh + d] = cvt<T>(v);
            } else {
              ((T*)a.v)[(((size_t)seq * a.heads + h) * a.npad + pos) * a.dh + d] = cvt<T>(v);
            }
          }
        }
      }
    } else if constexpr (EPI == EPI_GLU) {
      // tiles j (even) hold values, j+1 the gates of the same 16 features
      float* out = (float*)L.C + g.c_off0 + g.c_offb * (int64_t)M;
      const float* bias = L.bias + g.bias_off;
      const int T_ = L.glu_frames;
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const int colv = cb + j * 16 + l16;       // value column, gate column = colv + 16
        const int e = (colv >> 5) * 16 + l16;     // feature within the band
        if (colv >= g.N || e >= g.e1) continue;
        const float bv = bias[colv], bgt = bias[colv + 16];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rb + i * 16 + 4 * g4 + r;
            if (row >= M) continue;
            const int b = row / T_, t = row - b * T_;
            const float val = (acc[i][j][r] + bv) * sigmoidf_(acc[i][j + 1][r] + bgt);
            out[((int64_t)b * L.glu_total + g.e0 + e) * T_ + t] = val;
          }
        }
      }
    } else {
      const int64_t coff = g.c_off0 + g.c_offb * (int64_t)M;
      const float* bias = L.bias ? L.bias + g.bias_off : nullptr;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = cb + j * 16 + l16;
        if (col >= g.N) continue;
        const float bv = bias ? bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rb + i * 16 + 4 * g4 + r;
            if (row >= M) continue;
            const float v = acc[i][j][r] + bv;
            const int64_t idx = coff + (int64_t)row * L.ldc + col;
            if constexpr (EPI == EPI_EMBED) {
              ((float*)L.C)[idx] = v;
            } else if constexpr (EPI == EPI_RESID || EPI == EPI_FFN2) {
              ((float*)L.C)[idx] += v;
            } else if constexpr (EPI == EPI_GELU) {
              ((T*)L.C)[idx] = cvt<T>(gelu_erf(v));
            } else if constexpr (EPI == EPI_TANH) {
              ((T*)L.C)[idx] = cvt<T>(tanhf(v));
            }
          }
        }
      }
    }
  }

  __device__ static void run(const GemmLaunch& L) {
    __shared__ __attribute__((aligned(16))) char smem[2][(BM + BN) * kRowBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = L.M;
    GemmGroup g;
    int m0, n0;
    if (L.tiles) {
      const GemmTile t = L.tiles[blockIdx.x];
      g = L.groups[t.group];
      m0 = t.m0;
      n0 = t.n0;
    } else {
      g = L.dense;
      const int tn = (g.N + BN - 1) / BN;
      m0 = (blockIdx.x / tn) * BM;
      n0 = (blockIdx.x % tn) * BN;
    }
    if (m0 >= M) return;
    const char* A = (const char*)L.A + (g.a_off0 + g.a_offb * (int64_t)M) * (int64_t)sizeof(T);
    const char* B = (const char*)L.B + g.b_off * (int64_t)sizeof(T);
    const int K = g.K;
    const int64_t lda_b = (int64_t)g.lda * sizeof(T), ldb_b = (int64_t)g.ldb * sizeof(T);

    uint4 regs[PER];
    auto gload = [&](int k0) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int c = tid + p * kThreads;
        const int row = c >> 2, part = c & 3;
        const char* src;
        if (row < BM) {
          const int r = min(m0 + row, M - 1);
          src = A + r * lda_b;
        } else {
          const int r = min(n0 + row - BM, g.N - 1);
          src = B + r * ldb_b;
        }
        regs[p] = *(const uint4*)(src + (int64_t)k0 * sizeof(T) + part * 16);
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int c = tid + p * kThreads;
        const int row = c >> 2, part = c & 3;
        *(uint4*)(&smem[buf][row * kRowBytes + part * 16]) = regs[p];
      }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    gload(0);
    sstore(0);
    __syncthreads();
    const int a_row = wm * (BM / 2) + (lane & 15);
    const int b_row = BM + wn * (BN / 2) + (lane & 15);
    const int koff = (lane >> 4) * 16;
    int buf = 0;
    for (int k0 = 0; k0 < K; k0 += BK) {
      const bool more = k0 + BK < K;
      if (more) gload(k0 + BK);
      frag af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *(const frag*)(&smem[buf][(a_row + i * 16) * kRowBytes + koff]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = *(const frag*)(&smem[buf][(b_row + j * 16) * kRowBytes + koff]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma(acc[i][j], af[i], bf[j]);
      if (more) sstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    epilogue(L, g, M, m0 + wm * (BM / 2), n0 + wn * (BN / 2), acc, lane);
  }
};

template <typename T, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmLaunch L) {
  GemmKernel<T, EPI, 128, 128>::run(L);
}

template <typename T>
hipError_t launch_t(const GemmLaunch& L, hipStream_t stream) {
  int blocks;
  if (L.tiles) {
    blocks = L.n_tiles;
  } else {
    const int tm = (L.M + 127) / 128, tn = (L.dense.N + 127) / 128;
    blocks = tm * tn;
  }
  if (blocks <= 0) return hipSuccess;
  dim3 grid(blocks), block(kThreads);
  switch (L.epi) {
    case EPI_EMBED: hipLaunchKernelGGL((gemm_kernel<T, EPI_EMBED>), grid, block, 0, stream, L); break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<T, EPI_QKV>), grid, block, 0, stream, L); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_kernel<T, EPI_GELU>), grid, block, 0, stream, L); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<T, EPI_RESID>), grid, block, 0, stream, L); break;
    case EPI_TANH: hipLaunchKernelGGL((gemm_kernel<T, EPI_TANH>), grid, block, 0, stream, L); break;
    case EPI_GLU: hipLaunchKernelGGL((gemm_kernel<T, EPI_GLU>), grid, block, 0, stream, L); break;
    case EPI_FFN2: hipLaunchKernelGGL((gemm_kernel<T, EPI_FFN2>), grid, block, 0, stream, L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch& L, hipStream_t stream) {
  switch (L.dtype) {
    case DT_F32: return launch_t<float>(L, stream);
    case DT_F16: return launch_t<f16>(L, stream);
    case DT_BF16: return launch_t<bf16>(L, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mbr
