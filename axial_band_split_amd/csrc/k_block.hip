// The rest of a Transformer after its attention, in one kernel (fp16 / bf16):
//
//   x1 = x + o W_out^T                                    (o: gated attention output)
//   x2 = x1 + GELU(RMSNorm_f(x1) W_1^T + b_1) W_2^T + b_2
//   x3 = RMSNorm_out(x2)                                   -> X (fp32)
//   XH = x3 / max(|x3|, eps) * sqrt(D)   (the next attention's normalised input; its gain is in
//        the next W_qkv), or x3 itself after the last Transformer (the mask head's input)
//
// ([P1] "Per Attention layer", "The forward chain"; [P5] export-roformer.py classes Attn, FF and
// Block: the residual adds, the erf GELU feed-forward and the RMSNorm with its 1e-12 clamp.  The
// hidden layer holds twice the GELU, evaluated to 1.3e-4 by gelu2_tail (below the 16-bit rounding
// of the hidden layer), and the W_2 columns of the weight stream carry the factor 1/2, which is exact.)
//
// Tokens are the N side of every product: a wave owns 16 tokens and keeps, for all of them,
// the whole residual row in its accumulators (D/16 tiles of 16 x 16 on v_mfma_f32_16x16x32; lane
// l holds token l % 16 and rows 4(l/16) + v, v = 0..3, of each tile), so the norms are lane sums
// and two exchanges (lanes l ^ 16, l ^ 32), and neither x1 nor the FF-wide hidden layer ever leaves
// the registers:
//   * x1 feeds the first feed-forward product directly as its B operand: the columns of W_1 are
//     permuted once (at create) into the order in which the accumulators hold the rows;
//   * the hidden layer is produced 32 features at a time (two 16 x 16 tiles per wave), goes through
//     GELU in registers and is the B operand of the second product, whose K order is permuted the
//     same way;
//   * the second product accumulates onto x1 + b_2, so the residual add is free.
// The weights are one stream of equal stages (out-projection K steps of 64, then per 32 hidden
// features the W_1 rows of chunk c and the W_2 columns of chunk c-2), laid out at create in
// exactly the order the lanes read them: a stage is copied into LDS by 16-byte direct loads and
// every fragment read is one conflict-free 16-byte LDS read per lane.  Eight waves (128 tokens, two
// waves per SIMD, so one wave's products cover the other's LDS reads and vector work) share each
// stage; NS stages are in flight.
//
// Whole device passes (one 128-token block per compute unit) run every hidden chunk in
// each block.  The tokens left after them would leave most compute units idle for a full block's
// time, so they run in blocks that each take one group of hidden chunks (the out-projection is
// repeated per group), placed after the passes' blocks in the same grid so that they start on the
// compute units the last pass frees: each writes its part of the feed-forward sum (plus x1 in
// group 0), and a small kernel adds the parts, b_2, and applies the two norms.
#include <type_traits>

#include "kcommon.h"
#include "kernels.h"

namespace mbr {

namespace {


template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

constexpr int kMaxTailGroups = 32;   // chunk groups of the tail at most (block_part_bytes)

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

// fn(integral_constant<i>) for i = 0 .. N-1 (a loop whose index can select template arguments)
template <typename Fn, int... i>
__device__ __forceinline__ void static_for_impl(Fn fn, std::integer_sequence<int, i...>) {
  (fn(std::integral_constant<int, i>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn fn) { static_for_impl(fn, std::make_integer_sequence<int, N>{}); }

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

template <typename T, int D_, int I_, int NS_, int GS_, int VPM_>
struct BlockCfg {
  // GS: fragments per read group; VPM: vector instructions placed after each feed-forward product
  static constexpr int D = D_, I = I_, NS = NS_, GS = GS_, VPM = VPM_;
  static constexpr int WAVES = 8, THREADS = 64 * WAVES;
  static constexpr int DT = D / 16;                 // accumulator tiles per wave
  static constexpr int FF = 4 * D;
  static constexpr int NCH = FF / 32;               // hidden chunks of 32 features
  static constexpr int KO = I / 64;                 // out-projection stages (K = 64 each)
  static constexpr int NST = KO + NCH + 2;          // stages in the stream
  // stage bytes: D/8 fragments of 1 KB (out-projection: 2 K steps x D/16 tiles; feed-forward:
  // 2 W_1 tiles x D/32 K steps, then D/16 tiles of W_2)
  static constexpr int SB = D * 128;
  static constexpr int R = SB / (16 * THREADS);     // 16-byte loads per thread per stage
  static constexpr int LDS = NS * SB;               // the ring (b_1 is a static LDS array)
  static_assert(R * 16 * THREADS == SB, "stage split");
};

template <typename T, typename C, bool ALL_CHUNKS>
__device__ __forceinline__ void block_body(const BlockLaunch& L, const int bid, float* b1s) {
  typedef typename Frag<T>::type frag;
  constexpr int D = C::D, I = C::I, NS = C::NS, DT = C::DT, NCH = C::NCH, KO = C::KO, NST = C::NST,
                SB = C::SB, R = C::R, FF = C::FF, GS = C::GS, TH = C::THREADS;
  auto none = [](auto) {};
  extern __shared__ __attribute__((aligned(16))) char smem[];   // the weight ring

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qd = lane >> 4;
  // block = (token group, chunk group q); a wave owns 16 tokens of the group's 128 and runs the
  // hidden chunks [c0, c0 + n) (n even, at least 2).  With ALL_CHUNKS (the whole passes) the
  // block runs every chunk and the trip counts are compile-time constants.
  const int groups = ALL_CHUNKS ? 1 : L.groups;
  const int q = ALL_CHUNKS ? 0 : bid % groups;
  const int n = ALL_CHUNKS ? NCH : NCH / groups, c0 = q * n;
  const int64_t token = (ALL_CHUNKS ? 0 : L.tok0) + (int64_t)(bid / groups) * 128 + w * 16 + (lane & 15);
  const bool valid = token < L.tokens;
  // lanes past the last token read the last token's row and store nothing (a token's lanes only
  // ever combine with each other)
  const int64_t tload = valid ? token : (int64_t)L.tokens - 1;

  for (int i = tid; i < FF; i += TH) b1s[i] = L.b1[i];
  __syncthreads();

  const int wu = __builtin_amdgcn_readfirstlane(w);   // wave-uniform: LDS bases stay scalar
  // the weight stream as a buffer (NST * SB bytes; loads past the end would read zeros)
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(L.stream, NST * SB);
  // Step i of the block reads stream stage i (out-projection, i < KO) or KO + c0 + (i - KO) (the
  // stage holding W_1 of chunk c0 + i - KO and W_2 of the chunk two before it) into ring slot i % NS.
  const int nsteps = KO + n + 2;
  static_assert(NST == KO + NCH + 2, "stream length");
  auto issue = [&](int i) {
    const int g = (i < KO ? i : i + c0) * SB;
    char* l = smem + (i % NS) * SB + wu * 1024;
#pragma unroll
    for (int r = 0; r < R; ++r) buffer_dma16(srs, tid * 16, g + r * 16 * TH, l + r * 16 * TH);
  };
  // step i's stage is complete once at most (stages issued after it) * R loads are outstanding (the
  // attention-output loads issued in between only make this wait longer than needed).  With three
  // stages the stage two ahead is requested once this step's LDS reads are all issued; with two,
  // the next stage is requested right after the barrier, so that it has a whole step to arrive.
  // Either way its slot was last read in the previous step, which every wave finished before the
  // barrier.
  auto stage_begin = [&](int i) {
    if (i + NS - 2 < nsteps) wait_vm<(NS - 2) * R>();
    else wait_vm<0>();
    block_barrier();
    if constexpr (NS == 2) {
      if (i + 1 < nsteps) issue(i + 1);
    }
  };
  auto stage_end = [&](int i) {
    if constexpr (NS != 2) {
      if (i + NS - 1 < nsteps) issue(i + NS - 1);
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);

  // ---- x1 = x + o W_out^T; the attention output is read as B operands one stage ahead.  The
  // accumulators start at zero and x (fp32, DT 16-byte loads per lane) arrives in KO parts, part p
  // requested after stage p-1's weights and added at the start of stage p+2 (the last two after
  // the loop): every block of a device pass starts at once, and waiting for the whole residual
  // before the first product would expose one chip-wide burst of reads per pass.
  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[t][v] = 0.f;
  constexpr int XP = DT / KO;   // 16-byte residual loads per part
  static_assert(XP * KO == DT, "residual parts");
  const float* xr = L.X + tload * D + 4 * qd;
  float4 xs[3][XP];
  // residual piece t holds accumulator tile t (features 16t + 4(l/16) .. +3)
  // the wait counts below assume this issue order: keep the compiler from moving loads across
  auto order = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_x = [&](auto p_) {
    constexpr int p = decltype(p_)::value;
    order();
#pragma unroll
    for (int i = 0; i < XP; ++i) xs[p % 3][i] = *(const float4*)(xr + 16 * (p * XP + i));
  };
  auto add_x = [&](auto p_) {
    constexpr int p = decltype(p_)::value;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int t = p * XP + i;
      acc[t][0] += xs[p % 3][i].x;
      acc[t][1] += xs[p % 3][i].y;
      acc[t][2] += xs[p % 3][i].z;
      acc[t][3] += xs[p % 3][i].w;
    }
  };
  // the attention output of the lane's token, K elements 8(l/16) .. +7 of each 32-wide K step
  const T* orow = (const T*)L.O + tload * I + 8 * qd;
  frag ob[2][2];
  order();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) ob[0][ks] = *(const frag*)(orow + 32 * ks);
  load_x(std::integral_constant<int, 0>{});
  // loads issued after stage st's weights when stage st begins.  Three stages (two in flight): the
  // weights of stage 1, o of stage 0 and residual part 0 for st = 0; those plus stage 0's o,
  // weights and part for st = 1; then the part after the weights of st, and stage st-1's o, weights
  // and part.  Two stages (one in flight, the next requested right after the barrier): the o and the
  // residual part of the stage, issued after its weights.
  static_assert(NS == 2 || NS == 3, "ring depth");
  auto wait_outproj = [&](auto st_) {
    constexpr int st = decltype(st_)::value;
    constexpr int N = NS == 3 ? (st == 0 ? R + 2 + XP : st == 1 ? R + 4 + 2 * XP : R + 2 + 2 * XP) : 2 + XP;
    static_assert(N < 64, "vmcnt range");
    wait_vm<N>();
    block_barrier();
    if constexpr (NS == 2) issue(st + 1);
  };
  static_for<KO>([&](auto st_) {
    constexpr int st = decltype(st_)::value;
    wait_outproj(st_);
    if constexpr (st + 1 < KO)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) ob[(st + 1) & 1][ks] = *(const frag*)(orow + 64 * (st + 1) + 32 * ks);
    if constexpr (st >= 2) add_x(std::integral_constant<int, st - 2>{});
    const char* sl = smem + (st % NS) * SB + lane * 16;
    // fragment f = ks * DT + t
    pipelined<2 * DT, GS, 0, frag>([&](int f) { return *(const frag*)(sl + f * 1024); },
                                   [&](int f, const frag& a) { mma(acc[f % DT], a, ob[st & 1][f / DT]); }, none);
    stage_end(st);
    if constexpr (st + 1 < KO) load_x(std::integral_constant<int, st + 1>{});
  });
  add_x(std::integral_constant<int, KO - 2>{});
  add_x(std::integral_constant<int, KO - 1>{});

  // ---- RMSNorm_f(x1) as B operands (the gain is in W_1): K step s takes, in lane group l/16,
  // tiles 2s and 2s+1 (features 32s + 16(e/4) + 4(l/16) + e%4 for element e)
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) ss = fmaf(acc[t][v], acc[t][v], ss);
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  const float r1 = sqrtf((float)D) / fmaxf(sqrtf(ss), kNormEps);
  frag xb[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) xb[s][e] = cvt<T>(acc[2 * s + e / 4][e & 3] * r1);
  if (q != 0) {   // only chunk group 0 carries x1; the others accumulate their chunks' part
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[t][v] = 0.f;
  }

  // ---- feed-forward onto x1, three chunks in flight: step c (stage KO + c, holding the W_1 rows
  // of chunk c and the W_2 columns of chunk c - 2) runs chunk c's first product, the GELU of chunk
  // c-1's hidden tiles and chunk c-2's second product, all independent of each other, so the GELU's
  // vector work fills the shadows of the products.  The loop is unrolled by two so the hidden-tile
  // registers alternate without copies.
  constexpr int N1 = D / 16, N2 = DT;
  f32x4 hA[2] = {}, hB[2] = {};
  frag gA{}, gB{};
  auto step = [&](auto do1_, auto dog_, auto do2_, const char* sl, int c, f32x4 (&n0)[2], const f32x4 (&o0)[2],
                  frag& mk, const frag& us) {
    constexpr bool do1 = decltype(do1_)::value, dog = decltype(dog_)::value, do2 = decltype(do2_)::value;
    constexpr int NA = do1 ? N1 : 0, NB = do2 ? N2 : 0, G = (NA + NB) / GS;
    if constexpr (do1) {
      // the first product starts from b_1 (hidden features 32c + 16u + 4(l/16) + v of tile u), read
      // before any fragment so that waiting for it never waits for those
      const float* bb = b1s + 32 * c + 4 * qd;
      n0[0] = *(const f32x4*)bb;
      n0[1] = *(const f32x4*)(bb + 16);
    }
    // fragment f of the stage: W_1 tile f % 2, K step f / 2 (consecutive products go to different
    // accumulators), then W_2 tile f - N1
    auto rd = [&](int f) { return *(const frag*)(sl + (NA ? f : f + N1) * 1024); };
    auto mm = [&](int f, const frag& a) {
      if (f < NA) mma(n0[f & 1], a, xb[f >> 1]);
      else mma(acc[f - NA], a, us);
    };
    // twice the GELU of value e of the lane's 8 (hidden features 16(e/4) + 4(l/16) + e%4 of chunk
    // c-1) in region 1 + e G / 8 (all in "region 1" when there are no products)
    auto hook = [&](auto g_) {
      constexpr int g = decltype(g_)::value;
      if constexpr (dog) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (G == 0 || 1 + e * G / 8 == g) mk[e] = cvt<T>(gelu2_tail(o0[e >> 2][e & 3]));
      }
    };
    if constexpr (NA + NB == 0) {
      hook(std::integral_constant<int, 1>{});
    } else {
      pipelined<NA + NB, GS, C::VPM, frag>(rd, mm, hook);
    }
  };
  using Y = std::true_type;
  using Nn = std::false_type;
  // local step j (chunk c0 + j's first product, the GELU of the chunk before it, the second
  // product of the chunk two before it) with the register roles of its parity
  auto run = [&](auto d1, auto dg, auto d2, int j, f32x4 (&n0)[2], const f32x4 (&o0)[2], frag& mk, const frag& us) {
    const char* sl = smem + ((KO + j) % NS) * SB + lane * 16;
    step(d1, dg, d2, sl, c0 + j, n0, o0, mk, us);
  };
  // j = 0, 1
  stage_begin(KO);
  run(Y{}, Nn{}, Nn{}, 0, hA, hB, gA, gB);
  stage_end(KO);
  stage_begin(KO + 1);
  run(Y{}, Y{}, Nn{}, 1, hB, hA, gA, gB);
  stage_end(KO + 1);
  for (int j = 2; j < n; j += 2) {
    stage_begin(KO + j);
    run(Y{}, Y{}, Y{}, j, hA, hB, gB, gA);
    stage_end(KO + j);
    stage_begin(KO + j + 1);
    run(Y{}, Y{}, Y{}, j + 1, hB, hA, gA, gB);
    stage_end(KO + j + 1);
  }
  stage_begin(KO + n);
  run(Nn{}, Y{}, Y{}, n, hA, hB, gB, gA);
  stage_end(KO + n);
  stage_begin(KO + n + 1);
  run(Nn{}, Nn{}, Y{}, n + 1, hA, hB, gA, gB);

  if (!ALL_CHUNKS && groups > 1) {   // this group's part of x2 - b_2, for the reduction kernel
    if (!valid) return;
    float* pw = L.part + ((int64_t)q * (L.tokens - L.tok0) + (token - L.tok0)) * D + 4 * qd;
#pragma unroll
    for (int t = 0; t < DT; ++t) *(float4*)(pw + 16 * t) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    return;
  }

  // ---- x2 = acc + b_2;  x3 = RMSNorm_out(x2) -> X;  XH = x3 normalised (or x3)
  {
    const float* b2 = L.b2 + 4 * qd;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const f32x4 b = *(const f32x4*)(b2 + 16 * t);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += b[i];
    }
  }
  ss = 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) ss = fmaf(acc[t][v], acc[t][v], ss);
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  const float r2 = 1.0f / fmaxf(sqrtf(ss), kNormEps);
  const float* go = L.gout + 4 * qd;
  float ss3 = 0.f;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const f32x4 g = *(const f32x4*)(go + 16 * t);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] *= r2 * g[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) ss3 = fmaf(acc[t][i], acc[t][i], ss3);
  }
  ss3 += __shfl_xor(ss3, 16, 64);
  ss3 += __shfl_xor(ss3, 32, 64);
  const float r3 = L.xh_norm ? sqrtf((float)D) / fmaxf(sqrtf(ss3), kNormEps) : 1.0f;
  if (!valid) return;
  float* xw = L.X + token * D + 4 * qd;
  T* hw = (T*)L.XH + token * D + 4 * qd;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    *(float4*)(xw + 16 * t) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    typename Vec4<T>::type h4;
#pragma unroll
    for (int i = 0; i < 4; ++i) h4[i] = cvt<T>(acc[t][i] * r3);
    *(typename Vec4<T>::type*)(hw + 16 * t) = h4;
  }
}

// The whole device passes' blocks first, then the tail's (token group, chunk group) blocks, which
// start on the compute units the last pass frees.
template <typename T, typename C>
__global__ __launch_bounds__(C::THREADS, 2) void block_kernel(BlockLaunch L) {
  __shared__ __attribute__((aligned(16))) float b1s[C::FF];   // b_1, a separate LDS object
  if ((int)blockIdx.x < L.main_blocks) block_body<T, C, true>(L, blockIdx.x, b1s);
  else block_body<T, C, false>(L, blockIdx.x - L.main_blocks, b1s);
}

// x2 = b_2 + the chunk groups' parts (group 0 holds x1), then the epilogue of block_kernel:
// x3 = RMSNorm_out(x2) -> X, XH = x3 normalised (or x3).  One wave per token, lane l holding
// columns 2l, 2l + 1 of each 128-column slice.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_reduce_kernel(BlockLaunch L) {
  constexpr int P = D / 128;
  const int lane = threadIdx.x & 63;
  const int64_t ntail = (int64_t)L.tokens - L.tok0;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= ntail) return;
  float2 x[P];
#pragma unroll
  for (int k = 0; k < P; ++k) x[k] = *(const float2*)(L.b2 + 128 * k + 2 * lane);
#pragma unroll 8
  for (int q = 0; q < L.groups; ++q) {
    const float* pr = L.part + ((int64_t)q * ntail + r) * D + 2 * lane;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const float2 v = *(const float2*)(pr + 128 * k);
      x[k].x += v.x;
      x[k].y += v.y;
    }
  }
  auto wave_sum = [](float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
  };
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < P; ++k) ss = fmaf(x[k].y, x[k].y, fmaf(x[k].x, x[k].x, ss));
  const float r2 = 1.0f / fmaxf(sqrtf(wave_sum(ss)), kNormEps);
  float ss3 = 0.f;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const float2 g = *(const float2*)(L.gout + 128 * k + 2 * lane);
    x[k].x *= r2 * g.x;
    x[k].y *= r2 * g.y;
    ss3 = fmaf(x[k].y, x[k].y, fmaf(x[k].x, x[k].x, ss3));
  }
  const float r3 = L.xh_norm ? sqrtf((float)D) / fmaxf(sqrtf(wave_sum(ss3)), kNormEps) : 1.0f;
  const int64_t token = L.tok0 + r;
  float* xw = L.X + token * D + 2 * lane;
  T* hw = (T*)L.XH + token * D + 2 * lane;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    *(float2*)(xw + 128 * k) = x[k];
    hw[128 * k] = cvt<T>(x[k].x * r3);
    hw[128 * k + 1] = cvt<T>(x[k].y * r3);
  }
}

// chunk groups per 128-token group of the tail: the most that keep the tail within one device pass
// and split the nch hidden chunks into even runs (a block's loop takes its chunks two at a time)
int tail_groups(int64_t tail_blocks, int ncu, int nch) {
  int g = 1;
  for (int cand = 2; cand <= kMaxTailGroups; ++cand)
    if (nch % cand == 0 && (nch / cand) % 2 == 0 && tail_blocks * cand <= ncu) g = cand;
  return g;
}

template <typename T, typename C>
hipError_t launch_t(const BlockLaunch& L0, hipStream_t stream) {
  static_assert(C::NCH % 2 == 0, "the hidden chunks go two at a time");
  if (L0.ncu < 1 || L0.tokens < 1) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)block_kernel<T, C>, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (e != hipSuccess) return e;
  const int64_t pass = (int64_t)128 * L0.ncu, rest = L0.tokens % pass;
  BlockLaunch L = L0;
  // whole passes: 128 tokens and every hidden chunk to a block
  L.main_blocks = (int32_t)((L0.tokens - rest) / 128);
  // the tail: (token group, chunk group) blocks, partial sums reduced by block_reduce_kernel
  const int64_t tb = (rest + 127) / 128;
  L.tok0 = L0.tokens - rest;
  L.groups = rest ? tail_groups(tb, L0.ncu, C::NCH) : 1;
  if (L.groups > 1 && (!L.part || (size_t)L.groups * rest * C::D * 4 > block_part_bytes(C::D, L0.tokens, L0.ncu)))
    return hipErrorInvalidValue;
  const int64_t blocks = L.main_blocks + tb * L.groups;
  hipLaunchKernelGGL((block_kernel<T, C>), dim3((unsigned)blocks), dim3(C::THREADS), C::LDS, stream, L);
  if ((e = hipGetLastError()) != hipSuccess || rest == 0 || L.groups == 1) return e;
  hipLaunchKernelGGL((block_reduce_kernel<T, C::D>), dim3((unsigned)((rest + 3) / 4)), dim3(256), 0, stream, L);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const BlockLaunch& L, hipStream_t stream) {
  // LDS reads in groups of 3 fragments, 4 vector instructions after each feed-forward product (group
  // sizes 2, 3, 4 and 2, 4, 8 vector instructions time within 1%; 6 fragments about 1.5% slower)
  if (L.D == 384 && L.I == 512) return launch_t<T, BlockCfg<T, 384, 512, 3, 3, 4>>(L, stream);
  // D = 512: two stages of 64 KB (three would take 192 KB of LDS), read groups of 2
  if (L.D == 512 && L.I == 512) return launch_t<T, BlockCfg<T, 512, 512, 2, 2, 4>>(L, stream);
  return hipErrorInvalidValue;
}

}  // namespace

bool block_supported(int dtype, int D, int I, int FF) {
  return dtype != DT_F32 && FF == 4 * D && I == 512 && (D == 384 || D == 512);
}

size_t block_part_bytes(int D, int64_t tokens, int ncu) {
  const int64_t tail = std::min<int64_t>((int64_t)128 * ncu, kMaxTailGroups * ((tokens + 127) / 128 * 128));
  return (size_t)tail * D * 4;
}

int64_t block_stream_elems(int D, int I, int FF) {
  return (int64_t)(I / 64 + FF / 32 + 2) * D * 64;
}

hipError_t launch_block(const BlockLaunch& L, hipStream_t stream) {
  if (!block_supported(L.dtype, L.D, L.I, 4 * L.D)) return hipErrorInvalidValue;
  return L.dtype == DT_F16 ? launch_dt<f16>(L, stream) : launch_dt<bf16>(L, stream);
}

}  // namespace mbr
