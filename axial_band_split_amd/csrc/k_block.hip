// The rest of a Transformer after its attention, in one kernel (fp16 / bf16):
//
//   x1 = x + o W_out^T                                    (o: gated attention output)
//   x2 = x1 + GELU(RMSNorm_f(x1) W_1^T + b_1) W_2^T + b_2
//   x3 = RMSNorm_out(x2)                                   -> X (fp32)
//   XH = x3 / max(|x3|, eps) * sqrt(D)   (the next attention's normalised input; its gain is in
//        the next W_qkv), or x3 itself after the last Transformer (the mask head's input)
//
// ([P1] "Per Attention layer", "The forward chain"; [P5] export-roformer.py classes Attn, FF and
// Block: the residual adds, the exact-erf GELU feed-forward and the RMSNorm with its 1e-12 clamp.)
//
// Tokens are the N side of every product: a wave owns 32 tokens and keeps, for all of them,
// the whole residual row in its accumulators (D/32 tiles of 32 x 32 on v_mfma_f32_32x32x16; lane
// l holds token l % 32 and rows 8(v/4) + 4(l/32) + v%4 of each tile), so the norms are lane sums
// and one exchange with lane l ^ 32, and neither x1 nor the FF-wide hidden layer ever leaves the
// registers:
//   * x1 feeds the first feed-forward product directly as its B operand: the columns of W_1 are
//     permuted once (at create) into the order in which the accumulator holds the rows;
//   * the hidden layer is produced 32 features at a time (a 32 x 32 tile per wave), goes through
//     GELU in registers and is the B operand of the second product, whose K order is permuted the
//     same way;
//   * the second product accumulates onto x1 + b_2, so the residual add is free.
// The weights are one stream of equal stages (out-projection K steps of 64, then per 32 hidden
// features the W_1 rows of chunk c and the W_2 columns of chunk c-1), laid out at create in
// exactly the order the lanes read them: a stage is copied into LDS by 16-byte direct loads and
// every fragment read is one conflict-free 16-byte LDS read per lane.  Four waves (128 tokens)
// share each stage; NS stages are in flight.
#include <type_traits>

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

__device__ __forceinline__ void dma16(const char* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// A run of N products whose A fragments come from LDS, software-pipelined by hand: with one wave
// per SIMD the wave issues in order and every stall is exposed, so
//   region 0:      reads of group 0 (GS fragments)
//   region g >= 1: reads of group g (double-buffered in registers), the products of group g-1,
//                  and hook(g)'s vector work interleaved with those products
// with a scheduling fence after each region (otherwise the compiler hoists every read to the top,
// which needs N fragments of registers) and scheduling groups inside it (reads first, then one
// product and up to VPM vector instructions at a time).
template <typename Fn, int... g>
__device__ __forceinline__ void for_regions(Fn fn, std::integer_sequence<int, g...>) {
  (fn(std::integral_constant<int, g + 1>{}), ...);
}

template <int N, int GS, int VPM, typename F, typename RD, typename MM, typename HK>
__device__ __forceinline__ void pipelined(RD rd, MM mm, HK hook) {
  static_assert(N % GS == 0, "group size");
  constexpr int G = N / GS;
  F buf[2][GS];
#pragma unroll
  for (int j = 0; j < GS; ++j) buf[0][j] = rd(j);
  __builtin_amdgcn_sched_barrier(0);
  for_regions([&](auto g_) {
    constexpr int g = decltype(g_)::value;
    if constexpr (g < G) {
#pragma unroll
      for (int j = 0; j < GS; ++j) buf[g & 1][j] = rd(g * GS + j);
    }
#pragma unroll
    for (int j = 0; j < GS; ++j) mm((g - 1) * GS + j, buf[(g - 1) & 1][j]);
    hook(g_);
    if constexpr (g < G) __builtin_amdgcn_sched_group_barrier(0x100, GS, 0);
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (VPM > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }, std::make_integer_sequence<int, G>{});
}

template <typename T, int D_, int I_, int NS_, int GS_>
struct BlockCfg {
  static constexpr int D = D_, I = I_, NS = NS_, GS = GS_;   // GS: fragments per read group
  static constexpr int DT = D / 32;                 // accumulator tiles per wave
  static constexpr int FF = 4 * D;
  static constexpr int NCH = FF / 32;               // hidden chunks of 32 features
  static constexpr int KO = I / 64;                 // out-projection stages (K = 64 each)
  static constexpr int NST = KO + NCH + 2;          // stages in the stream
  // stage bytes: D/8 fragments of 1 KB (out-projection: 4 K steps x D/32 tiles; feed-forward:
  // D/16 K steps of W_1 + 2 K steps x D/32 tiles of W_2)
  static constexpr int SB = D * 128;
  static constexpr int R = SB / 4096;               // 16-byte loads per thread per stage
  static constexpr int LDS = NS * SB;               // the ring (b_1 is a static LDS array)
  static_assert(DT % 3 == 0 && 9 * 16 * 64 * 4 <= NS * SB, "split-block reduction layout");
};

template <typename T, typename C, bool SPLIT_BLOCKS>
__global__ __launch_bounds__(256, 1) void block_kernel(BlockLaunch L) {
  typedef typename Frag<T>::type frag;
  constexpr int D = C::D, I = C::I, NS = C::NS, DT = C::DT, NCH = C::NCH, KO = C::KO, NST = C::NST,
                SB = C::SB, R = C::R, FF = C::FF, GS = C::GS;
  auto none = [](auto) {};
  extern __shared__ __attribute__((aligned(16))) char smem[];   // the weight ring
  __shared__ __attribute__((aligned(16))) float b1s[FF];        // b_1, a separate LDS object

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5;
  // Blocks below split_from own 128 tokens (a strip of 32 per wave).  The blocks after them take
  // the tokens left over from whole rounds over the device one strip each: the four waves share
  // the strip and split the hidden chunks (wave w runs chunks c = w mod 4), then add their parts.
  constexpr bool split = SPLIT_BLOCKS;
  const int64_t token = split ? (int64_t)L.split_from * 128 + (int64_t)blockIdx.x * 32 + (lane & 31)
                              : (int64_t)blockIdx.x * 128 + w * 32 + (lane & 31);
  const bool valid = token < L.tokens;
  // lanes past the last token read the last token's row and store nothing (a token's lanes only
  // ever combine with each other)
  const int64_t tload = valid ? token : (int64_t)L.tokens - 1;
  const char* stream = (const char*)L.stream;

  for (int i = tid; i < FF; i += 256) b1s[i] = L.b1[i];
  __syncthreads();

  const int wu = __builtin_amdgcn_readfirstlane(w);   // wave-uniform: LDS bases stay scalar
  auto issue = [&](int st) {
    const char* g = stream + (size_t)st * SB + tid * 16;
    char* l = smem + (st % NS) * SB + wu * 1024;
#pragma unroll
    for (int r = 0; r < R; ++r) dma16(g + r * 4096, l + r * 4096);
  };
  // stage st is complete once at most (stages issued after it) * R loads are outstanding (the
  // attention-output loads issued in between only make this wait longer than needed).  The next
  // stage is requested once this one's LDS reads are all issued: its slot was last read in the
  // previous step, which every wave finished before the barrier.
  auto stage_begin = [&](int st) {
    if (st + NS - 2 < NST) wait_vm<(NS - 2) * R>();
    else wait_vm<0>();
    block_barrier();
  };
  auto stage_end = [&](int st) {
    if (st + NS - 1 < NST) issue(st + NS - 1);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);

  // x (fp32) straight into the accumulators
  f32x16 acc[DT];
  const float* xr = L.X + tload * D + 4 * h;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *(const float4*)(xr + 32 * t + 8 * j);
      acc[t][4 * j + 0] = v.x;
      acc[t][4 * j + 1] = v.y;
      acc[t][4 * j + 2] = v.z;
      acc[t][4 * j + 3] = v.w;
    }

  // ---- x1 = x + o W_out^T; the attention output is read as B operands one stage ahead
  const T* orow = (const T*)L.O + tload * I + 8 * h;
  frag ob[2][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) ob[0][ks] = *(const frag*)(orow + 16 * ks);
#pragma unroll
  for (int st = 0; st < KO; ++st) {
    stage_begin(st);
    if (st + 1 < KO)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ob[(st + 1) & 1][ks] = *(const frag*)(orow + 64 * (st + 1) + 16 * ks);
    const char* sl = smem + (st % NS) * SB + lane * 16;
    // fragment f = ks * DT + t
    pipelined<4 * DT, GS, 0, frag>([&](int f) { return *(const frag*)(sl + f * 1024); },
                                   [&](int f, const frag& a) { mma32(acc[f % DT], a, ob[st & 1][f / DT]); }, none);
    stage_end(st);
  }

  // ---- RMSNorm_f(x1) as B operands (the gain is in W_1)
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) ss = fmaf(acc[t][v], acc[t][v], ss);
  ss += __shfl_xor(ss, 32, 64);
  const float r1 = sqrtf((float)D) / fmaxf(sqrtf(ss), kNormEps);
  frag xb[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) xb[s][e] = cvt<T>(acc[s >> 1][8 * (s & 1) + e] * r1);
  if (split && w != 0) {   // only wave 0 carries x1; the others accumulate their hidden chunks' part
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
  }

  // ---- feed-forward onto x1, three chunks in flight: step c (stage KO + c, holding the W_1 rows
  // of chunk c and the W_2 columns of chunk c - 2) runs chunk c's first product, the GELU of chunk
  // c-1's hidden tile and chunk c-2's second product, all independent of each other, so the GELU's
  // vector work fills the shadows of the products.  The loop is unrolled by two so the hidden-tile
  // registers alternate without copies.  (A chain of dependent products on one accumulator runs
  // at full rate on this matrix core, so the first product needs only one.)
  constexpr bool SPLIT = false;
  constexpr int N1 = D / 16, N2 = 2 * DT;
  f32x16 hA0{}, hA1{}, hB0{}, hB1{};
  frag gA0{}, gA1{}, gB0{}, gB1{};
  auto step = [&](auto do1_, auto dog_, auto do2_, const char* sl, int c, f32x16& n0, f32x16& n1,
                  const f32x16& o0, const f32x16& o1, frag& mk0, frag& mk1, const frag& us0, const frag& us1) {
    constexpr bool do1 = decltype(do1_)::value, dog = decltype(dog_)::value, do2 = decltype(do2_)::value;
    constexpr int NA = do1 ? N1 : 0, NB = do2 ? N2 : 0, G = (NA + NB) / GS;
    if constexpr (do1) {
      // the first product starts from b_1 (rows 8(v/4) + 4h + v%4 of chunk c), read before any
      // fragment so that waiting for it never waits for those
      const float* bb = b1s + 32 * c + 4 * h;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 b = *(const f32x4*)(bb + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          n0[4 * j + i] = b[i];
          if constexpr (SPLIT) n1[4 * j + i] = 0.f;
        }
      }
    }
    // second-product fragment k = f - NA: tile k % DT, K step k / DT (consecutive products go to
    // different accumulators); the stream stores tile t's two K steps at 2t, 2t+1
    auto rd = [&](int f) {
      const int k = f - NA;
      return *(const frag*)(sl + (f < NA ? f : N1 + 2 * (k % DT) + k / DT) * 1024);
    };
    auto mm = [&](int f, const frag& a) {
      if (f < NA) {
        if (SPLIT && (f & 1)) mma32(n1, a, xb[f]);
        else mma32(n0, a, xb[f]);
      } else {
        const int k = f - NA;
        mma32(acc[k % DT], a, (k / DT) ? us1 : us0);
      }
    };
    // GELU value v of the lane's 16 (hidden rows 8(v/4) + 4h + v%4 of chunk c-1) in region
    // 1 + v G / 16 (all in "region 1" when there are no products)
    auto hook = [&](auto g_) {
      constexpr int g = decltype(g_)::value;
      if constexpr (dog) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (G == 0 || 1 + v * G / 16 == g) {
            const float y = SPLIT ? o0[v] + o1[v] : o0[v];
            (v < 8 ? mk0 : mk1)[v & 7] = cvt<T>(gelu_erf(y));
          }
      }
    };
    if constexpr (NA + NB == 0) {
      hook(std::integral_constant<int, 1>{});
    } else {
      pipelined<NA + NB, GS, 8, frag>(rd, mm, hook);
    }
  };
  using Y = std::true_type;
  using Nn = std::false_type;
  auto slot = [&](int c) { return smem + ((KO + c) % NS) * SB + lane * 16; };
  // step c with the register roles of its parity; in a split block, wave w does only the part of
  // the step that belongs to its chunks (first product of c, GELU of c-1 or second product of
  // c-2, whichever is w's; the block still meets at every stage)
  auto run = [&](auto d1, auto dg, auto d2, int c, f32x16& n0, f32x16& n1, const f32x16& o0, const f32x16& o1,
                 frag& mk0, frag& mk1, const frag& us0, const frag& us1) {
    constexpr bool D1 = decltype(d1)::value, DG = decltype(dg)::value, D2 = decltype(d2)::value;
    const char* sl = slot(c);
    if constexpr (!split) {
      step(d1, dg, d2, sl, c, n0, n1, o0, o1, mk0, mk1, us0, us1);
    } else {
      const int sel = (c - w) & 3;
      if (D1 && sel == 0) step(Y{}, Nn{}, Nn{}, sl, c, n0, n1, o0, o1, mk0, mk1, us0, us1);
      else if (DG && sel == 1) step(Nn{}, Y{}, Nn{}, sl, c, n0, n1, o0, o1, mk0, mk1, us0, us1);
      else if (D2 && sel == 2) step(Nn{}, Nn{}, Y{}, sl, c, n0, n1, o0, o1, mk0, mk1, us0, us1);
    }
  };
  // c = 0, 1
  stage_begin(KO);
  run(Y{}, Nn{}, Nn{}, 0, hA0, hA1, hB0, hB1, gA0, gA1, gB0, gB1);
  stage_end(KO);
  stage_begin(KO + 1);
  run(Y{}, Y{}, Nn{}, 1, hB0, hB1, hA0, hA1, gA0, gA1, gB0, gB1);
  stage_end(KO + 1);
  for (int c = 2; c < NCH; c += 2) {
    stage_begin(KO + c);
    run(Y{}, Y{}, Y{}, c, hA0, hA1, hB0, hB1, gB0, gB1, gA0, gA1);
    stage_end(KO + c);
    stage_begin(KO + c + 1);
    run(Y{}, Y{}, Y{}, c + 1, hB0, hB1, hA0, hA1, gA0, gA1, gB0, gB1);
    stage_end(KO + c + 1);
  }
  stage_begin(KO + NCH);
  run(Nn{}, Y{}, Y{}, NCH, hA0, hA1, hB0, hB1, gB0, gB1, gA0, gA1);
  stage_end(KO + NCH);
  stage_begin(KO + NCH + 1);
  run(Nn{}, Nn{}, Y{}, NCH + 1, hA0, hA1, hB0, hB1, gA0, gA1, gB0, gB1);

  if constexpr (split) {
    // wave 0 adds the other waves' parts, three tiles per wave at a time through the (now idle)
    // ring: lane-consecutive floats, [wave-1][tile][v][lane]
    float* red = (float*)smem;
#pragma unroll
    for (int p = 0; p < DT / 3; ++p) {
      block_barrier();
      if (w != 0) {
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int v = 0; v < 16; ++v) red[(((w - 1) * 3 + q) * 16 + v) * 64 + lane] = acc[3 * p + q][v];
      }
      __syncthreads();
      if (w == 0) {
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
          for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[3 * p + q][v] += red[((u * 3 + q) * 16 + v) * 64 + lane];
      }
    }
    if (w != 0) return;
  }

  // ---- x2 = acc + b_2;  x3 = RMSNorm_out(x2) -> X;  XH = x3 normalised (or x3)
  {
    const float* b2 = L.b2 + 4 * h;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 b = *(const f32x4*)(b2 + 32 * t + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][4 * j + i] += b[i];
      }
  }
  ss = 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) ss = fmaf(acc[t][v], acc[t][v], ss);
  ss += __shfl_xor(ss, 32, 64);
  const float r2 = 1.0f / fmaxf(sqrtf(ss), kNormEps);
  const float* go = L.gout + 4 * h;
  float ss3 = 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 g = *(const f32x4*)(go + 32 * t + 8 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][4 * j + i] *= r2 * g[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) ss3 = fmaf(acc[t][4 * j + i], acc[t][4 * j + i], ss3);
    }
  ss3 += __shfl_xor(ss3, 32, 64);
  const float r3 = L.xh_norm ? sqrtf((float)D) / fmaxf(sqrtf(ss3), kNormEps) : 1.0f;
  if (!valid) return;
  float* xw = L.X + token * D + 4 * h;
  T* hw = (T*)L.XH + token * D + 4 * h;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *(float4*)(xw + 32 * t + 8 * j) = make_float4(acc[t][4 * j], acc[t][4 * j + 1], acc[t][4 * j + 2], acc[t][4 * j + 3]);
      typename Vec4<T>::type q;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = cvt<T>(acc[t][4 * j + i] * r3);
      *(typename Vec4<T>::type*)(hw + 32 * t + 8 * j) = q;
    }
}

template <typename T, typename C>
hipError_t launch_t(const BlockLaunch& L, hipStream_t stream) {
  // the last 128-token block may be partial only when no strips follow it
  if (L.split_from < 0 || (int64_t)L.split_from * 128 >= (int64_t)L.tokens + 128) return hipErrorInvalidValue;
  // blocks of 128 tokens, then one 32-token strip per block for the rest
  if (L.split_from > 0) {
    hipError_t e = hipFuncSetAttribute((const void*)block_kernel<T, C, false>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((block_kernel<T, C, false>), dim3(L.split_from), dim3(256), C::LDS, stream, L);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t rest = (int64_t)L.tokens - (int64_t)L.split_from * 128;
  const int strips = rest > 0 ? (int)((rest + 31) / 32) : 0;
  if (strips > 0) {
    hipError_t e = hipFuncSetAttribute((const void*)block_kernel<T, C, true>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((block_kernel<T, C, true>), dim3(strips), dim3(256), C::LDS, stream, L);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_dt(const BlockLaunch& L, hipStream_t stream) {
  if (L.D == 384 && L.I == 512) return launch_t<T, BlockCfg<T, 384, 512, 3, 8>>(L, stream);
  return hipErrorInvalidValue;
}

}  // namespace

// D = 512 fits the registers only with spills in the feed-forward loop; that width keeps the
// separate products.
bool block_supported(int dtype, int D, int I, int FF) {
  return dtype != DT_F32 && FF == 4 * D && I == 512 && D == 384;
}

int64_t block_stream_elems(int D, int I, int FF) {
  return (int64_t)(I / 64 + FF / 32 + 2) * D * 64;
}

hipError_t launch_block(const BlockLaunch& L, hipStream_t stream) {
  if (!block_supported(L.dtype, L.D, L.I, 4 * L.D)) return hipErrorInvalidValue;
  return L.dtype == DT_F16 ? launch_dt<f16>(L, stream) : launch_dt<bf16>(L, stream);
}

}  // namespace mbr
