// Axial attention of the core: softmax(q k^T * scale) v per (sequence, head), times the head's
// gate, written back in token layout ([P1] "Per Attention layer": per-head sigmoid gates on the
// attention output; [P5] export-roformer.py class Attn).
//
// q, k and v arrive as [seq][head][position][dh].  Both kernels compute the transposed products
// S^T = K Q^T and O^T = V^T P^T on the matrix cores; V is transposed while it is staged in LDS.
// In the 16 x 16 accumulator layout a lane then owns one query column, so the softmax statistics
// of a query (running max, running sum) and the rescaling of its output stay in that lane's
// registers; only the max needs a reduction over the four lane groups of the wave.  The
// probabilities leave the S^T accumulators directly as the B operand of the P.V product: for
// 16-bit types the 8 keys a lane feeds are the 4 + 4 keys it holds in two neighbouring S^T tiles,
// and the V^T operand is read with the same key order.
//
//   time axis (n = frames, up to thousands): flash loop over 64-key tiles staged in LDS and
//   shared by the 4 waves of a workgroup, online softmax in fp32 (exp2 with log2(e) folded into
//   the score scale); the [seqs, H, n, n] scores never exist in memory ([P3] "How these graphs are
//   written" shows why: 1110 MiB of scores at 1100 frames).
//   band axis (n = bands <= 64): one wave per (sequence, head), all keys in one tile, operands
//   straight from global memory (there is nothing to share between waves).
#include "kcommon.h"
#include "kernels.h"

namespace mbr {

namespace {

constexpr float kNegBig = -1e30f;

// P (fp32 probabilities in S^T accumulator layout) to the B operand of one P.V step.
template <typename T>
struct PFrag {
  // 16-bit: one step covers 32 keys = S^T tiles 2m and 2m+1
  static constexpr int KEYS = 32;
  typedef typename Frag<T>::type type;
  __device__ static type make(const f32x4& lo, const f32x4& hi) {
    type f;
    f[0] = cvt<T>(lo[0]); f[1] = cvt<T>(lo[1]); f[2] = cvt<T>(lo[2]); f[3] = cvt<T>(lo[3]);
    f[4] = cvt<T>(hi[0]); f[5] = cvt<T>(hi[1]); f[6] = cvt<T>(hi[2]); f[7] = cvt<T>(hi[3]);
    return f;
  }
  // V^T operand: row d of a [dh][keys] tile at byte address `row`, keys of step m in lane group g
  __device__ static type vload(const char* row, int m, int g4) {
    type f;
    typedef typename Frag<T>::half_type h4;
    const h4 a = *(const h4*)(row + (32 * m + 4 * g4) * sizeof(T));
    const h4 b = *(const h4*)(row + (32 * m + 16 + 4 * g4) * sizeof(T));
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
  }
};
template <>
struct PFrag<float> {
  // fp32: one step covers 16 keys = one S^T tile, already in the B layout
  static constexpr int KEYS = 16;
  typedef f32x4 type;
  __device__ static type make(const f32x4& lo, const f32x4&) { return lo; }
  __device__ static type vload(const char* row, int m, int g4) {
    return *(const f32x4*)(row + (16 * m + 4 * g4) * sizeof(float));
  }
};

// ---------------------------------------------------------------------------------- time axis
// grid (npad/128, H, seqs), 256 threads; wave w owns queries blockIdx.x*128 + 32w .. +31.
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_time_kernel(AttnLaunch L) {
  constexpr int EPF = Frag<T>::EPF;
  constexpr int KS = 4 * EPF;                 // head dims per matrix-core step
  constexpr int DSTEPS = DH / KS;
  constexpr int KT = 64;                      // keys per tile
  constexpr int KROW = DH * (int)sizeof(T) + 16;
  constexpr int VROW = KT * (int)sizeof(T) + 16;
  constexpr int PV = KT / PFrag<T>::KEYS;     // P.V steps per key tile
  constexpr int SPP = PFrag<T>::KEYS / 16;    // S^T tiles per P.V step
  using frag = typename Frag<T>::type;
  __shared__ __attribute__((aligned(16))) char lds[KT * KROW + DH * VROW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int h = blockIdx.y, seq = blockIdx.z;
  const int n = L.n, npad = L.npad;
  const int q0 = blockIdx.x * 128 + wave * 32;
  const size_t base = ((size_t)seq * L.heads + h) * (size_t)npad * DH;
  const T* Q = (const T*)L.q + base;
  const T* K = (const T*)L.k + base;
  const T* V = (const T*)L.v + base;

  frag qf[2][DSTEPS];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) qf[c][s] = *(const frag*)(Q + (size_t)(q0 + c * 16 + l16) * DH + s * KS + g4 * EPF);

  f32x4 oacc[DH / 16][2];
#pragma unroll
  for (int d = 0; d < DH / 16; ++d) oacc[d][0] = oacc[d][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {kNegBig, kNegBig}, lrun[2] = {0.f, 0.f};

  const int ntiles = (n + KT - 1) / KT;
  for (int kt = 0; kt < ntiles; ++kt) {
    constexpr int KCH = DH * (int)sizeof(T) / 16;
    for (int c = threadIdx.x; c < KT * KCH; c += 256) {
      const int r = c / KCH, p = c - r * KCH;
      *(uint4*)(lds + r * KROW + p * 16) = *(const uint4*)((const char*)(K + (size_t)(kt * KT + r) * DH) + p * 16);
    }
    // V tile [64 keys][DH] -> LDS as V^T [DH][keys]
    constexpr int EPC = 16 / (int)sizeof(T);
    constexpr int DCH = DH / EPC;
    for (int c = threadIdx.x; c < KT * DCH; c += 256) {
      const int r = c / DCH, p = c - r * DCH;
      const uint4 raw = *(const uint4*)(V + (size_t)(kt * KT + r) * DH + p * EPC);
      const T* vals = (const T*)&raw;
#pragma unroll
      for (int e = 0; e < EPC; ++e) *(T*)(lds + KT * KROW + (p * EPC + e) * VROW + r * (int)sizeof(T)) = vals[e];
    }
    __syncthreads();

    f32x4 s[4][2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r][0] = s[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) {
        const frag a = *(const frag*)(lds + (r * 16 + l16) * KROW + (st * KS + g4 * EPF) * (int)sizeof(T));
        mma(s[r][0], a, qf[0][st]);
        mma(s[r][1], a, qf[1][st]);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float mx = kNegBig;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kt * KT + r * 16 + 4 * g4 + e;
          const float v = key < n ? s[r][c][e] * L.scale_log2 : kNegBig;
          s[r][c][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrun[c], mx);
      const float alpha = exp2f(mrun[c] - mnew);
      mrun[c] = mnew;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = exp2f(s[r][c][e] - mnew);
          s[r][c][e] = p;
          sum += p;
        }
      lrun[c] = lrun[c] * alpha + sum;
#pragma unroll
      for (int d = 0; d < DH / 16; ++d) oacc[d][c] *= alpha;
    }
#pragma unroll
    for (int m = 0; m < PV; ++m) {
      typename PFrag<T>::type pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) pf[c] = PFrag<T>::make(s[m * SPP][c], s[m * SPP + SPP - 1][c]);
#pragma unroll
      for (int d = 0; d < DH / 16; ++d) {
        const auto a = PFrag<T>::vload(lds + KT * KROW + (d * 16 + l16) * VROW, m, g4);
        mma(oacc[d][0], a, pf[0]);
        mma(oacc[d][1], a, pf[1]);
      }
    }
    __syncthreads();
  }

  const int I = L.heads * DH;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float l = lrun[c];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int q = q0 + c * 16 + l16;
    if (q >= n) continue;
    const size_t row = (size_t)seq * L.frames + q;
    const float scale = L.gates[row * L.heads + h] / l;
    T* dst = (T*)L.o + row * I + h * DH + 4 * g4;
#pragma unroll
    for (int d = 0; d < DH / 16; ++d) {
      typename Vec4<T>::type o4;   // 4 consecutive dims: one 8-byte (16-byte for fp32) store
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = cvt<T>(oacc[d][c][e] * scale);
      *(typename Vec4<T>::type*)(dst + d * 16) = o4;
    }
  }
}

// ---------------------------------------------------------------------------------- band axis
// One wave per (sequence, head); grid ceil(seqs*H / 4), 256 threads.  n <= 64 = npad.
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_band_kernel(AttnLaunch L) {
  constexpr int EPF = Frag<T>::EPF;
  constexpr int KS = 4 * EPF;
  constexpr int DSTEPS = DH / KS;
  constexpr int PV = 64 / PFrag<T>::KEYS;
  constexpr int SPP = PFrag<T>::KEYS / 16;
  using frag = typename Frag<T>::type;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int sh = blockIdx.x * 4 + wave;
  if (sh >= L.seqs * L.heads) return;
  const int seq = sh / L.heads, h = sh - seq * L.heads;
  const int n = L.n;
  const size_t base = (size_t)sh * 64 * DH;
  const T* Q = (const T*)L.q + base;
  const T* K = (const T*)L.k + base;
  const T* V = (const T*)L.v + base;
  constexpr int VROW = 64 * (int)sizeof(T) + 16;
  __shared__ __attribute__((aligned(16))) char vlds_all[4][DH * VROW];
  char* vlds = vlds_all[wave];
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int DCH = DH / EPC;
  const int I = L.heads * DH;
  const int BT = L.batch * L.frames;
  // Softmax over the keys, P.V and the gated store of the 16 queries of column block c, from their
  // S^T tiles sc[r] (keys 16r .. 16r + 15).  One block at a time keeps 32 accumulator registers
  // live instead of 128, which leaves room for more waves per SIMD.
  auto column = [&](int c, f32x4 (&sc)[4]) {
    float mx = kNegBig;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = r * 16 + 4 * g4 + e;
        const float v = key < n ? sc[r][e] * L.scale_log2 : kNegBig;
        sc[r][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(sc[r][e] - mx);
        sc[r][e] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    f32x4 oacc[DH / 16];
#pragma unroll
    for (int d = 0; d < DH / 16; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < PV; ++m) {
      const typename PFrag<T>::type pf = PFrag<T>::make(sc[m * SPP], sc[m * SPP + SPP - 1]);
#pragma unroll
      for (int d = 0; d < DH / 16; ++d) mma(oacc[d], PFrag<T>::vload(vlds + (d * 16 + l16) * VROW, m, g4), pf);
    }
    const int q = c * 16 + l16;
    if (q >= n) return;
    const size_t row = (size_t)q * BT + seq;
    const float scale = L.gates[row * L.heads + h] / sum;
    T* dst = (T*)L.o + row * I + h * DH + 4 * g4;
#pragma unroll
    for (int d = 0; d < DH / 16; ++d) {
      typename Vec4<T>::type o4;   // 4 consecutive dims: one 8-byte (16-byte for fp32) store
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = cvt<T>(oacc[d][e] * scale);
      *(typename Vec4<T>::type*)(dst + d * 16) = o4;
    }
  };
  if constexpr (sizeof(T) == 2) {
    // Every load of the wave is issued before the first is used (one memory round trip): V four
    // keys x 8 dims per lane and pass, then the Q and K fragments of every K step.
    constexpr int VP = (64 / 4) * DCH / 64;
    static_assert((64 / 4) * DCH % 64 == 0, "whole passes");
    uint4 vraw[VP][4];
#pragma unroll
    for (int it = 0; it < VP; ++it) {
      const int idx = it * 64 + lane, kg = idx / DCH, p = idx - kg * DCH;
#pragma unroll
      for (int j = 0; j < 4; ++j) vraw[it][j] = *(const uint4*)(V + (size_t)(4 * kg + j) * DH + p * EPC);
    }
    frag qf[DSTEPS][4], kf[DSTEPS][4];
#pragma unroll
    for (int st = 0; st < DSTEPS; ++st)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qf[st][c] = *(const frag*)(Q + (size_t)(c * 16 + l16) * DH + st * KS + g4 * EPF);
        kf[st][c] = *(const frag*)(K + (size_t)(c * 16 + l16) * DH + st * KS + g4 * EPF);
      }
    // V [64 keys][DH] -> V^T [DH][keys] in the wave's own LDS slice: (4 keys) x 1 dim per 8-byte write
#pragma unroll
    for (int it = 0; it < VP; ++it) {
      const int idx = it * 64 + lane, kg = idx / DCH, p = idx - kg * DCH;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        typename Vec4<T>::type k4;
#pragma unroll
        for (int j = 0; j < 4; ++j) k4[j] = ((const T*)&vraw[it][j])[e];
        *(typename Vec4<T>::type*)(vlds + (p * EPC + e) * VROW + 4 * kg * (int)sizeof(T)) = k4;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x4 sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) mma(sc[r], kf[st][r], qf[st][c]);
      column(c, sc);
    }
  } else {
    f32x4 s[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) s[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this wave's V [64 keys][DH] -> V^T [DH][keys] in its own LDS slice
    for (int c = lane; c < 64 * DCH; c += 64) {
      const int r = c / DCH, p = c - r * DCH;
      const uint4 raw = *(const uint4*)(V + (size_t)r * DH + p * EPC);
      const T* vals = (const T*)&raw;
#pragma unroll
      for (int e = 0; e < EPC; ++e) *(T*)(vlds + (p * EPC + e) * VROW + r * (int)sizeof(T)) = vals[e];
    }
#pragma unroll
    for (int st = 0; st < DSTEPS; ++st) {
      frag qf[4], kf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[c] = *(const frag*)(Q + (size_t)(c * 16 + l16) * DH + st * KS + g4 * EPF);
#pragma unroll
      for (int r = 0; r < 4; ++r) kf[r] = *(const frag*)(K + (size_t)(r * 16 + l16) * DH + st * KS + g4 * EPF);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) mma(s[r][c], kf[r], qf[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x4 sc[4] = {s[0][c], s[1][c], s[2][c], s[3][c]};
      column(c, sc);
    }
  }
}

template <typename T, int DH>
hipError_t launch_dh(const AttnLaunch& L, hipStream_t stream) {
  if (L.axis == 0) {
    dim3 grid(L.npad / 128, L.heads, L.seqs);
    hipLaunchKernelGGL((attn_time_kernel<T, DH>), grid, dim3(256), 0, stream, L);
  } else {
    dim3 grid((L.seqs * L.heads + 3) / 4);
    hipLaunchKernelGGL((attn_band_kernel<T, DH>), grid, dim3(256), 0, stream, L);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnLaunch& L, hipStream_t stream) {
  if (L.dh == 64) return launch_dh<T, 64>(L, stream);
  if (L.dh == 32) return launch_dh<T, 32>(L, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& L, hipStream_t stream) {
  if (L.axis == 0 && L.npad % 128) return hipErrorInvalidValue;
  if (L.axis == 1 && (L.npad != 64 || L.n > 64)) return hipErrorInvalidValue;
  switch (L.dtype) {
    case DT_F32: return launch_t<float>(L, stream);
    case DT_F16: return launch_t<f16>(L, stream);
    case DT_BF16: return launch_t<bf16>(L, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mbr
