// MFMA GEMM for 16-bit operands (fp16 / bf16) on gfx950: C = A . B^T with fused epilogues.
//
// Same problems and epilogues as the generic family (k_gemm.hip) — the linear layers of the core
// ([P1] "Per Attention layer", "Parameter accounting"; [P5] export-roformer.py classes Attn, FF and
// the mask MLP) — laid out for the CDNA4 matrix cores:
//   * 256 x 128 block tile, 4 waves of 128 x 64, v_mfma_f32_32x32x16 (each lane feeds 16 bytes of
//     A and of B per 32 x 32 x 16 product, half the operand traffic of the 16 x 16 shape);
//   * K in steps of 32 elements (64-byte rows) through a 3-stage LDS ring filled by 16-byte direct
//     global->LDS loads, two stages in flight while the third is consumed; each wave waits for its
//     own loads with s_waitcnt and the workgroup meets at one barrier per step;
//   * rows are stored with their four 16-byte chunks XOR-permuted by ((row>>1) ^ (row>>2)) & 3 so
//     the 32 rows one fragment read touches fall on distinct LDS banks;
//   * dense launches walk the tiles so that each XCD (workgroups are dealt round-robin to the 8
//     XCDs) receives one contiguous run of tiles: neighbouring tiles share their A panel in that
//     XCD's L2;
//   * the epilogue stages each wave's accumulators through LDS and writes 16-byte vectors: rows of
//     q, k, v (rotary applied to the pairs a lane already holds), GELU / tanh outputs, fp32
//     residual updates, and the GLU of paired 32-feature value / gate blocks stored feature-major.
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

constexpr int BM = 256, BN = 128, NS = 3, ROWB = 64;
constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
constexpr int A_LD = A_BYTES / (256 * 16), B_LD = B_BYTES / (256 * 16);
constexpr int LOADS = A_LD + B_LD;  // 16-byte loads per thread per stage (= 6)
static_assert(LOADS == 6, "the s_waitcnt immediates below assume 6 loads per stage");
constexpr int EP_STRIDE = 68;                   // floats per staged row (64 + 4: keeps 16-B alignment)
constexpr int EP_WAVE = 64 * EP_STRIDE * 4;     // bytes of one wave's staging area (64 rows)
constexpr int LDS_BYTES = NS * STAGE;
static_assert(4 * EP_WAVE <= LDS_BYTES, "epilogue staging fits in the ring");

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ void dma16(const char* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <typename T> struct Pack8;
template <> struct Pack8<f16> { typedef f16x8 type; };
template <> struct Pack8<bf16> { typedef bf16x8 type; };

template <typename T, int EPI>
__global__ __launch_bounds__(256, 2) void gemm2_kernel(GemmLaunch L) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using frag = typename Frag<T>::type;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
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
    const int nb = gridDim.x, per = nb >> 3, rem = nb & 7;
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int logical = x * per + min(x, rem) + slot;
    const int tn = (g.N + BN - 1) / BN;
    m0 = (logical / tn) * BM;
    n0 = (logical % tn) * BN;
  }
  if (m0 >= M) return;

  // ---- loader: thread's 16-byte chunks of every stage (global source, wave-uniform LDS target)
  const char* Ag = (const char*)L.A + (g.a_off0 + g.a_offb * (int64_t)M) * 2;
  const char* Bg = (const char*)L.B + g.b_off * 2;
  const int64_t lda_b = (int64_t)g.lda * 2, ldb_b = (int64_t)g.ldb * 2;
  const char* src[LOADS];
  int dst[LOADS];
#pragma unroll
  for (int j = 0; j < A_LD; ++j) {
    const int row = (j * 4 + w) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    src[j] = Ag + (int64_t)min(m0 + row, M - 1) * lda_b + c * 16;
    dst[j] = (j * 4 + w) * 1024;
  }
#pragma unroll
  for (int j = 0; j < B_LD; ++j) {
    const int row = (j * 4 + w) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    src[A_LD + j] = Bg + (int64_t)min(n0 + row, g.N - 1) * ldb_b + c * 16;
    dst[A_LD + j] = A_BYTES + (j * 4 + w) * 1024;
  }
  auto issue = [&](int ks) {
    char* base = smem + (ks % NS) * STAGE;
    const int64_t ko = (int64_t)ks * 64;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) dma16(src[j] + ko, base + dst[j]);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = g.K >> 5;
  issue(0);
  if (nk > 1) issue(1);
  const int r32 = lane & 31, khalf = lane >> 5;
  for (int kk = 0; kk < nk; ++kk) {
    if (kk + 1 < nk) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    if (kk + 2 < nk) issue(kk + 2);
    const char* st = smem + (kk % NS) * STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 2 * ks + khalf;
      frag a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r32;
        a[i] = *(const frag*)(st + row * ROWB + ((c ^ swz(row)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + r32;
        b[j] = *(const frag*)(st + A_BYTES + row * ROWB + ((c ^ swz(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma32(acc[i][j], a[i], b[j]);
    }
  }

  // ---- epilogue: every wave is done with the ring once all have passed this barrier
  asm volatile("s_barrier" ::: "memory");
  const int cbase = n0 + wn * 64;
  if (cbase >= g.N) return;
  float* ep = (float*)(smem + w * EP_WAVE);
  const float* bias = L.bias ? L.bias + g.bias_off : nullptr;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = ii * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
          ep[r * EP_STRIDE + j * 32 + r32] = acc[2 * half + ii][j][v];
        }
    const int rbase = m0 + wm * 128 + half * 64;
    if constexpr (EPI == EPI_RESID || EPI == EPI_EMBED) {
      // fp32 rows of 64 columns: 16 lanes x 4 floats per row, 4 rows per pass
      const int c4 = (lane & 15) * 4;
      float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bias) bv = *(const float4*)(bias + cbase + c4);
      float* C = (float*)L.C + g.c_off0 + g.c_offb * (int64_t)M;
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int row = rbase + r;
        if (row >= M) continue;
        const float4 a = *(const float4*)(ep + r * EP_STRIDE + c4);
        float4* o = (float4*)(C + (int64_t)row * L.ldc + cbase + c4);
        float4 val = make_float4(a.x + bv.x, a.y + bv.y, a.z + bv.z, a.w + bv.w);
        if constexpr (EPI == EPI_RESID) {
          const float4 x = *o;
          val = make_float4(x.x + val.x, x.y + val.y, x.z + val.z, x.w + val.w);
        }
        *o = val;
      }
    } else if constexpr (EPI == EPI_GLU) {
      // 32 value columns then their 32 gate columns; lane = row, loop over features
      float* out = (float*)L.C + g.c_off0 + g.c_offb * (int64_t)M;
      const int row = rbase + lane;
      const int T_ = L.glu_frames;
      const int b = row / T_, t = row - b * T_;
      const int fbase = (cbase >> 6) * 32;
#pragma unroll 4
      for (int e = 0; e < 32; ++e) {
        if (fbase + e >= g.e1) break;
        const float val = (ep[lane * EP_STRIDE + e] + bias[cbase + e]) *
                          sigmoidf_(ep[lane * EP_STRIDE + 32 + e] + bias[cbase + 32 + e]);
        if (row < M) out[((int64_t)b * L.glu_total + g.e0 + fbase + e) * T_ + t] = val;
      }
    } else {
      // 16-bit rows of 64 columns: 8 lanes x 8 elements per row, 8 rows per pass
      typedef typename Pack8<T>::type pack;
      const int c8 = (lane & 7) * 8;
      float bvals[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bvals[e] = bias ? bias[cbase + c8 + e] : 0.f;
      int which = 0, h = 0, d0 = 0;
      const QkvArgs& qa = L.qkv;
      if constexpr (EPI == EPI_QKV) {
        const int I = qa.heads * qa.dh;
        which = cbase / I;
        const int f = cbase + c8 - which * I;
        h = f / qa.dh;
        d0 = f - h * qa.dh;
      }
      if constexpr (EPI == EPI_QKV) {
        if (which == 2 && qa.axis == 0) {
          // time axis: v goes out transposed, [seq][h][dh][npad]; lane = row, so every store
          // instruction writes 64 consecutive positions of one head dimension
          const int row = rbase + lane;
          if (row < M) {
            const int seq = row / qa.frames, pos = row - seq * qa.frames;
            T* vt = (T*)qa.v + (size_t)seq * qa.heads * qa.dh * qa.npad + pos;
            const int f0 = cbase - 2 * qa.heads * qa.dh;   // v feature of this wave's first column
#pragma unroll 8
            for (int d = 0; d < 64; ++d) {
              // feature f = h * dh + dd sits at row (h * dh + dd) of the [H*dh][npad] block of seq
              vt[(size_t)(f0 + d) * qa.npad] = cvt<T>(ep[lane * EP_STRIDE + d]);
            }
          }
          continue;
        }
      }
#pragma unroll 2
      for (int it = 0; it < 8; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int row = rbase + r;
        if (row >= M) continue;
        const float4 a0 = *(const float4*)(ep + r * EP_STRIDE + c8);
        const float4 a1 = *(const float4*)(ep + r * EP_STRIDE + c8 + 4);
        float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        pack p;
        if constexpr (EPI == EPI_QKV) {
          int seq, pos;
          if (qa.axis == 0) {
            seq = row / qa.frames;
            pos = row - seq * qa.frames;
          } else {
            const int BT = qa.batch * qa.frames;
            pos = row / BT;
            seq = row - pos * BT;
          }
          if (which < 2) {
            const float4 cs = *(const float4*)(qa.cos + pos * (qa.dh >> 1) + (d0 >> 1));
            const float4 sn = *(const float4*)(qa.sin + pos * (qa.dh >> 1) + (d0 >> 1));
            const float cc[4] = {cs.x, cs.y, cs.z, cs.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x0 = v[2 * q], x1 = v[2 * q + 1];
              v[2 * q] = x0 * cc[q] - x1 * ss[q];
              v[2 * q + 1] = x0 * ss[q] + x1 * cc[q];
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = cvt<T>(v[e]);
          T* dstp = (T*)(which == 0 ? qa.q : which == 1 ? qa.k : qa.v);
          *(pack*)(dstp + (((size_t)seq * qa.heads + h) * qa.npad + pos) * qa.dh + d0) = p;
        } else {
          T* C = (T*)L.C + g.c_off0 + g.c_offb * (int64_t)M;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = v[e] + bvals[e];
            if constexpr (EPI == EPI_GELU) p[e] = cvt<T>(gelu_erf(x));
            else p[e] = cvt<T>(tanhf(x));
          }
          *(pack*)(C + (int64_t)row * L.ldc + cbase + c8) = p;
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_t(const GemmLaunch& L, hipStream_t stream) {
  int blocks;
  if (L.tiles) {
    blocks = L.n_tiles;
  } else {
    if (L.dense.N % 64 || L.dense.K % 32) return hipErrorInvalidValue;
    blocks = ((L.M + BM - 1) / BM) * ((L.dense.N + BN - 1) / BN);
  }
  if (blocks <= 0) return hipSuccess;
  dim3 grid(blocks), block(256);
#define GEMM2_CASE(E)                                                                                  \
  case E: {                                                                                            \
    static bool attr = false;                                                                          \
    if (!attr) {                                                                                       \
      hipError_t e = hipFuncSetAttribute((const void*)gemm2_kernel<T, E>,                              \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);       \
      if (e != hipSuccess) return e;                                                                   \
      attr = true;                                                                                     \
    }                                                                                                  \
    hipLaunchKernelGGL((gemm2_kernel<T, E>), grid, block, LDS_BYTES, stream, L);                       \
    break;                                                                                             \
  }
  switch (L.epi) {
    GEMM2_CASE(EPI_EMBED)
    GEMM2_CASE(EPI_QKV)
    GEMM2_CASE(EPI_GELU)
    GEMM2_CASE(EPI_RESID)
    GEMM2_CASE(EPI_TANH)
    GEMM2_CASE(EPI_GLU)
    default: return hipErrorInvalidValue;
  }
#undef GEMM2_CASE
  return hipGetLastError();
}

}  // namespace

int gemm2_tile_rows() { return BM; }

hipError_t launch_gemm2(const GemmLaunch& L, hipStream_t stream) {
  switch (L.dtype) {
    case DT_F16: return launch_t<f16>(L, stream);
    case DT_BF16: return launch_t<bf16>(L, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mbr
