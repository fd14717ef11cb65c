// The band-axis attention of a Transformer in one kernel (fp16 / bf16): the q, k, v projection of
// one head for the bands of a few frames, the attention over the bands of each frame, and the gated
// output, with q, k and v never leaving the compute unit.
//
// ([P1] "The two transformers are not the same shape": the band Transformer runs one sequence per
// frame over the bands, positions = band index; "Per Attention layer": x^ W_qkv^T split head-major,
// rotary on q and k, softmax(q k^T / sqrt(dh)) v per head, times sigmoid(x^ W_g^T + b_g) per head.
// The scale 1/sqrt(dh) is folded into W_q at create; q is multiplied by log2 e here so the
// exponentials are base 2.)
//
// Workgroup = (FR frames, head h), two waves per frame (FR = 2).  The FR x 64 band slots of the
// frames (bands >= NB are padding rows, read as a valid row and masked as keys) are the rows of a
// 64 FR x 192 x D product
// against the head's rows of W_qkv ([q_h | k_h | v_h]); K goes through a 2-stage LDS ring by 16-byte
// direct loads, as in the GEMM (the next step's loads in flight during each step; three workgroups
// per compute unit hide the rest of the latency).  Wave (f, r) owns the 32 band slots 32r .. 32r+31 of frame f and all
// 192 columns (six 32 x 32 tiles on v_mfma_f32_32x32x16):
//   * the q and k tiles are taken transposed (features x tokens), so a lane holds one token and four
//     consecutive features per group: the rotary pairs are in the lane, and the accumulator read in
//     8-element halves is directly an operand of the score product S^T = K Q^T (the feature order
//     inside each 16-feature step is permuted the same way for q and k, which a dot product allows);
//   * the v tiles are taken as tokens x features, which read the same way are the V^T operand of
//     O^T = V^T P^T whose key order matches the probabilities straight from the S^T accumulators;
//   * the two waves of a frame swap their keys' k and v fragments through LDS (8 KB each);
//   * the gate of each token is a dot product on the vector units over the A fragments the product
//     already holds (two lanes per token, half the K step each; packed 16-bit dot instructions with
//     fp32 accumulation).
// The softmax runs over one tile of 64 keys (the 60 bands of a frame) in registers; the output goes
// out through a per-wave LDS staging as 16-byte rows.
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

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// sum_e a[e] b[e] + c over eight 16-bit pairs: the products are exact in fp32
__device__ __forceinline__ float dot8(const f16x8& a, const f16x8& b, float c) {
  typedef f16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_fdot2(h2{a[2 * i], a[2 * i + 1]}, h2{b[2 * i], b[2 * i + 1]}, c, false);
  return c;
}
__device__ __forceinline__ float dot8(const bf16x8& a, const bf16x8& b, float c) {
  typedef bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_fdot2_f32_bf16(b2{a[2 * i], a[2 * i + 1]}, b2{b[2 * i], b[2 * i + 1]}, c, false);
  return c;
}

// 16-byte chunks of a 64-byte LDS row, XOR-permuted so the 32 rows of a fragment read spread over
// the banks (the GEMM's layout)
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

constexpr float kNegBig = -1e30f;

// FR frames per workgroup, two waves per frame
template <int FR>
struct BandCfg {
  static constexpr int kRows = 64 * FR;                  // FR frames x 64 band slots
  static constexpr int kCols = 192;                      // [q_h | k_h | v_h], dh = 64
  static constexpr int kWaves = 2 * FR, kThreads = 64 * kWaves;
  static constexpr int kStage = (kRows + kCols) * 64;    // one K step of 32
  static constexpr int kNS = 2;
  static constexpr int kOcc = 3;                         // workgroups per compute unit (LDS, VGPRs)
  static constexpr int kExch = kWaves * 8192;            // per wave: its keys' 4 k and 4 v fragments
  static constexpr int kOut = kWaves * 4096;             // per wave: 32 tokens x 64 outputs, 16-bit
  static constexpr int kLds = (kNS * kStage > kExch + kOut ? kNS * kStage : kExch + kOut);
  // past the ring, free until the output staging: the gate weights (D <= 1024, 16-bit) and the
  // rotary rows of positions 0..7 and 0, 8, .., 56
  static constexpr int kAux = kNS * kStage;
  static_assert(kAux + 8192 <= kLds, "auxiliary tables fit past the ring");
  static constexpr int kALoads = kRows * 4 / kThreads;   // 16-byte A loads per thread per stage (2)
  static constexpr int kBChunks = kCols * 4;             // 768
  static constexpr int kBLoads = (kBChunks + kThreads - 1) / kThreads;
  static_assert(kALoads * kThreads == kRows * 4, "A loads");
};

template <typename T, int FR>
__global__ __launch_bounds__(128 * FR, BandCfg<FR>::kOcc) void band_attn_kernel(BandLaunch L) {
  using C = BandCfg<FR>;
  constexpr int kRows = C::kRows, kCols = C::kCols, kStage = C::kStage, kNS = C::kNS, kExch = C::kExch,
                NT = C::kThreads, NW = C::kWaves;
  using frag = typename Frag<T>::type;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int r32 = lane & 31, hl = lane >> 5;
  const int fl = wu >> 1, half = wu & 1;                    // frame of the group, band half
  const int D = L.D, I = L.heads * 64, BT = L.BT, NB = L.NB;
  // workgroups are dealt round-robin to the 8 XCDs: one contiguous run each, so the 8 heads of a
  // frame group (the same rows of x^) share an L2
  const int nb = gridDim.x, per = nb >> 3, rem = nb & 7;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int logical = xcd * per + min(xcd, rem) + slot;
  const int h = logical % L.heads, f0 = (logical / L.heads) * FR;

  T* wg = (T*)(smem + C::kAux);                             // the head's gate weights
  float4* rt = (float4*)(smem + C::kAux + 4096);            // [16][16]: (cos, sin) of pairs 2q, 2q+1
  for (int i = tid; i < D; i += NT) wg[i] = ((const T*)L.W)[(size_t)(3 * I + h) * D + i];
  for (int i = tid; i < 256; i += NT) {     // row r: position r (r < 8) or 8 (r - 8)
    const int r = i >> 4, q = i & 15, pos = r < 8 ? r : 8 * (r - 8);
    const float2 c = *(const float2*)(L.cos + pos * 32 + 2 * q);
    const float2 sn = *(const float2*)(L.sin + pos * 32 + 2 * q);
    rt[i] = make_float4(c.x, sn.x, c.y, sn.y);
  }
  __syncthreads();

  // ---- loader.  A row rho: frame f0 + rho/64, band slot rho%64 -> token slot*BT + frame (padding
  // rows read the nearest valid token); B row c: W_qkv row h*64 + c of q, k or v.
  const int64_t rowb = (int64_t)D * 2;
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc_uniform(L.XH, (uint32_t)((int64_t)NB * BT * rowb));
  const __amdgpu_buffer_rsrc_t brs = buffer_rsrc_uniform(L.W, (uint32_t)((int64_t)(3 * I + 64) * rowb));
  int voff[C::kALoads + C::kBLoads];
#pragma unroll
  for (int j = 0; j < C::kALoads; ++j) {   // A: 4 chunks per row
    const int c = j * NT + tid, row = c >> 2, pc = c & 3;
    const int f = min(f0 + (row >> 6), BT - 1), s = min(row & 63, NB - 1);
    voff[j] = (int)(((int64_t)s * BT + f) * rowb) + ((pc ^ swz(row)) << 4);
  }
#pragma unroll
  for (int j = 0; j < C::kBLoads; ++j) {   // B: 768 chunks (a partial last round covers the first waves)
    const int c = j * NT + tid, row = min(c >> 2, kCols - 1), pc = c & 3;
    const int wrow = (row >> 6) * I + h * 64 + (row & 63);
    voff[C::kALoads + j] = (int)(wrow * rowb) + ((pc ^ swz(row)) << 4);
  }
  // loads of this wave per stage (the partial last B round only for waves below its end)
  const bool blast = ((C::kBLoads - 1) * NT + wu * 64) < C::kBChunks;
  auto issue = [&](int ks) {
    char* base = smem + (ks % kNS) * kStage;
    const int ko = ks * 64;
#pragma unroll
    for (int j = 0; j < C::kALoads; ++j) buffer_dma16(ars, voff[j], ko, base + (j * NW + wu) * 1024);
#pragma unroll
    for (int j = 0; j < C::kBLoads; ++j)
      if (j < C::kBLoads - 1 || blast) buffer_dma16(brs, voff[C::kALoads + j], ko, base + kRows * 64 + (j * NW + wu) * 1024);
  };

  // ---- the 64 FR x 192 product; this wave: rows 64 fl + 32 half + (0..31), all six column tiles.
  // Tiles 0..3 (q, k) as C^T = W X^T, tiles 4, 5 (v) as C = X W^T.
  f32x16 acc[6];
#pragma unroll
  for (int j = 0; j < 6; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  float gdot = 0.f;                         // gate: this lane's token, K half hl of every step
  const int arow = 64 * fl + 32 * half + r32;
  const int nk = D >> 5;
  // row scale of this lane's token (x^ not yet normalised: sqrt(D) / |x|), its statistics read with
  // the first stage
  const int slot_me = 32 * half + r32;                  // this lane's band slot (token of tiles 0..3)
  const int fr = f0 + fl;
  const int64_t token = (int64_t)min(slot_me, NB - 1) * BT + min(fr, BT - 1);
  float4 rs[4];
  if (L.rowss) {
    const float4* p = (const float4*)(L.rowss + token * kSsStride);
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = p[i];
  }
  issue(0);
  wait_vm<0>();
  float sc = 1.0f;
  if (L.rowss) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += (rs[i].x + rs[i].y) + (rs[i].z + rs[i].w);
    sc = L.rs_mul / fmaxf(sqrtf(ss), kNormEps);
  }
  for (int ks = 0; ks < nk; ++ks) {
    if (ks) wait_vm<0>();                   // this wave's loads of step ks
    block_barrier();                        // everyone's; and every wave is done with step ks-1
    // the gate weights of this step, read before the next stage's loads are issued: an LDS read
    // after them that the compiler cannot tell apart from the ring would wait for those loads
    frag gw[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) gw[kh] = *(const frag*)(wg + ks * 32 + 8 * (2 * kh + hl));
    if (ks + 1 < nk) issue(ks + 1);         // into the slot of step ks-1
    const char* st = smem + (ks % kNS) * kStage;
    frag a[2], b[2][6];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int lc = 2 * kh + hl;
      a[kh] = *(const frag*)(st + arow * 64 + ((lc ^ swz(arow)) << 4));
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int brow = 32 * j + r32;
        b[kh][j] = *(const frag*)(st + kRows * 64 + brow * 64 + ((lc ^ swz(brow)) << 4));
      }
    }
    // gate: chunks hl and 2 + hl of this step for the lane's token, the A fragments
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) gdot = dot8(a[kh], gw[kh], gdot);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int j = 0; j < 4; ++j) mma32(acc[j], b[kh][j], a[kh]);
#pragma unroll
      for (int j = 4; j < 6; ++j) mma32(acc[j], a[kh], b[kh][j]);
    }
  }

  // ---- gate; rotary on q and k, q in log2 units
  gdot += __shfl_xor(gdot, 32, 64);
  const float gate = sigmoidf_(gdot * sc + L.gate_bias[h]);
  // q (tiles 0, 1) and k (tiles 2, 3): element v is feature 32 (j%2) + 8 (v/4) + 4 hl + v%4 of the token
  // slot_me; pairs (2p, 2p+1) are elements (4g, 4g+1), (4g+2, 4g+3)
  frag qf[4], kf[4];
  const float4* rhi = rt + (8 + (slot_me >> 3)) * 16;   // angles of slot 8 a + b = those of 8 a plus b
  const float4* rlo = rt + (slot_me & 7) * 16;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * jj + 8 * g4 + 4 * hl;
      const float4 hi = rhi[d >> 2], lo = rlo[d >> 2];
      const float2 cs = make_float2(hi.x * lo.x - hi.y * lo.y, hi.z * lo.z - hi.w * lo.w);
      const float2 sn = make_float2(hi.y * lo.x + hi.x * lo.y, hi.w * lo.z + hi.z * lo.w);
#pragma unroll
      for (int j = jj; j < 4; j += 2) {    // q tile jj, then k tile jj + 2
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[j][4 * g4 + e] * sc;
        float y[4];
        y[0] = x[0] * cs.x - x[1] * sn.x;
        y[1] = x[0] * sn.x + x[1] * cs.x;
        y[2] = x[2] * cs.y - x[3] * sn.y;
        y[3] = x[2] * sn.y + x[3] * cs.y;
        const float m = j < 2 ? L.q_mul : 1.0f;
        frag& dst = j < 2 ? qf[2 * jj + (g4 >> 1)] : kf[2 * jj + (g4 >> 1)];
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * (g4 & 1) + e] = cvt<T>(y[e] * m);
      }
      // two groups' rotary rows at a time: their results are made before the next groups' reads
      if (g4 & 1) asm volatile("" : "+v"(qf[2 * jj + (g4 >> 1)]), "+v"(kf[2 * jj + (g4 >> 1)]) :: "memory");
    }
  }
  // v (tiles 4, 5): lane = feature 32 (j-4) + r32, element v = token slot 32 half + 8 (v/4) + 4 hl + v%4:
  // the row scale of each element's token, from the lane holding that token
  frag vf[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float s = __shfl(sc, 8 * (v >> 2) + 4 * hl + (v & 3), 64);   // sc = 1 without statistics
      vf[j][v >> 3][v & 7] = cvt<T>(acc[4 + j][v] * s);
    }

  // ---- swap keys with the other half of the frame: this wave's k (as S^T A operand) and v (as V^T
  // A operand) fragments, 8 x 1 KB, lanes contiguous
  block_barrier();                          // every wave is done with the ring
  char* mine = smem + wu * 8192 + lane * 16;
  const char* theirs = smem + (wu ^ 1) * 8192 + lane * 16;
#pragma unroll
  for (int s = 0; s < 4; ++s) *(frag*)(mine + s * 1024) = kf[s];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int s = 0; s < 2; ++s) *(frag*)(mine + (4 + 2 * j + s) * 1024) = vf[j][s];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  block_barrier();
  frag kp[4], vp[2][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) kp[s] = *(const frag*)(theirs + s * 1024);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int s = 0; s < 2; ++s) vp[j][s] = *(const frag*)(theirs + (4 + 2 * j + s) * 1024);

  // ---- S^T (64 keys x this wave's 32 queries): key tile t holds the slots of half t
  f32x16 st[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int v = 0; v < 16; ++v) st[t][v] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) mma32(st[t], (t == half) ? kf[s] : kp[s], qf[s]);
  }
  // keys past the last band get probability 0; scores are in log2 units
  float mx = kNegBig;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = 32 * t + 8 * (v >> 2) + 4 * hl + (v & 3);
      if (key >= NB) st[t][v] = kNegBig;
      mx = fmaxf(mx, st[t][v]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float lsum = 0.f;
  frag pf[4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(st[t][v] - mx);
      lsum += p;
      pf[2 * t + (v >> 3)][v & 7] = cvt<T>(p);
    }
  lsum += __shfl_xor(lsum, 32, 64);
  // ---- O^T = V^T P^T: key step ks (16 keys) is half ks/2's v fragment ks%2
  f32x16 o[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int v = 0; v < 16; ++v) o[j][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) mma32(o[j], ((ks >> 1) == half) ? vf[j][ks & 1] : vp[j][ks & 1], pf[ks]);
  }

  // ---- gated output: stage [token][64] 16-bit rows per wave, then 16-byte stores of whole rows
  const float scale = gate / lsum;
  char* ob = smem + kExch + wu * 4096;
  static_assert(NW == 2 * FR, "two waves per frame");
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      typename Vec4<T>::type q4;
#pragma unroll
      for (int e = 0; e < 4; ++e) q4[e] = cvt<T>(o[j][4 * g4 + e] * scale);
      const int d = 32 * j + 8 * g4 + 4 * hl;
      *(typename Vec4<T>::type*)(ob + r32 * 128 + ((((d >> 3) ^ (r32 & 7)) << 4) | ((d & 4) << 1))) = q4;
    }
  // each lane's own staging rows only: the wave reads back what it wrote (in order, lgkmcnt)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int tk = it * 8 + (lane >> 3), c8 = lane & 7;    // token of the wave, 16-byte chunk
    const frag val = *(const frag*)(ob + tk * 128 + ((c8 ^ (tk & 7)) << 4));
    const int s = 32 * half + tk;
    if (fr < BT && s < NB) *(frag*)((T*)L.O + ((int64_t)s * BT + fr) * I + h * 64 + 8 * c8) = val;
  }
}

}  // namespace

namespace {
template <typename T, int FR>
hipError_t launch_fr(const BandLaunch& L, hipStream_t stream) {
  using C = BandCfg<FR>;
  const int groups = (L.BT + FR - 1) / FR;
  hipError_t e = hipFuncSetAttribute((const void*)band_attn_kernel<T, FR>, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((band_attn_kernel<T, FR>), dim3((unsigned)(groups * L.heads)), dim3(C::kThreads), C::kLds, stream, L);
  return hipGetLastError();
}
}  // namespace

bool band_attn_supported(int dtype, int NB, int heads, int dh, int D) {
  return dtype != DT_F32 && dh == 64 && NB >= 1 && NB <= 64 && heads >= 1 && D % 32 == 0 && D <= 1024;
}

hipError_t launch_band_attn(const BandLaunch& L, hipStream_t stream) {
  if (!band_attn_supported(L.dtype, L.NB, L.heads, 64, L.D) || L.BT < 1) return hipErrorInvalidValue;
  // two frames (four waves) per workgroup, three workgroups per compute unit: one's projection
  // overlaps the others' attention and load waits (0.86 ms per forward at 1100 frames; a 3-stage ring
  // with two workgroups per compute unit 0.94, four frames per workgroup 0.97, one frame 1.73)
  if (L.dtype == DT_F16) return launch_fr<f16, 2>(L, stream);
  return launch_fr<bf16, 2>(L, stream);
}

}  // namespace mbr
