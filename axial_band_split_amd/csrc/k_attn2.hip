// Time-axis attention for 16-bit operands on gfx950 (flash form, online softmax in fp32).
//
// One sequence is one (batch, band) pair of the time Transformer, its positions the frames
// ([P1] "The two transformers are not the same shape"); per head, o = softmax(q k^T) v with the
// 1/sqrt(dh) scale already folded into W_q and q scaled by log2(e) by the projection's epilogue
// (scores in log2 units), times the head's gate ([P1] "Per Attention layer").
//
//   * workgroup = 4 waves x 32 queries; the K tile [64 keys][dh] and the V^T tile [dh][64 keys]
//     (V^T is written that way by the q/k/v projection) arrive by 16-byte direct global->LDS loads
//     into a 2-stage ring, the next tile in flight while the current one is consumed;
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16: a lane owns one query column and 16 of
//     the 32 keys of a tile, so a query's max needs one exchange with the lane 32 apart; the S^T
//     accumulators start at minus the running reference, so a probability is one exponential; a
//     lane adds up the probabilities it holds as rounded to 16 bits (the values the P.V product
//     uses), two per packed dot instruction against ones with fp32 accumulation (the matrix core,
//     already the busier unit, would spend a quarter more products on a ones-row sum at dh = 64);
//   * the probabilities feed the P.V product straight from the S^T accumulators: the K rows of the
//     S^T product are taken in a permuted order so that the 8 probabilities a lane holds for one
//     16-key step belong to 8 consecutive keys, and the matching V^T operand is one 16-byte read;
//   * the reference used for the exponentials is the first tile's max.  A later tile's
//     exponentials are taken against it without looking at the tile's max; only when a lane's sum
//     of them passes 2^12 (so one of them passed 2^7) is the tile's max taken, and the reference
//     raised when that max exceeds it by more than 8 (log2 units), the accumulators rescaled and
//     the exponentials taken again.  Any reference value gives the same softmax; the bounds keep
//     every exponential that reaches the products <= 2^12, far inside the 16-bit range;
//   * rows of 128 bytes hold their 16-byte chunks XOR-permuted by (row >> 1) & 7, so the rows one
//     fragment read touches spread over all LDS banks;
//   * only the last key tile is masked (keys >= n), and the workgroup order keeps all query blocks of
//     one (sequence, head) on one XCD, whose L2 then serves its K and V;
//   * the q / k width DQK and the v width DV are separate template parameters: an attention whose
//     queries and keys are twice as deep as its values (the polar positional scheme of [P2]
//     "Evaluation record", section "BS PolarFormer...", part "Ported, and what it actually bought",
//     which asks for a fused attention that accepts v narrower than q) runs in the same loop.
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

// d = a b + c with c kept (a separate accumulator input)
__device__ __forceinline__ f32x16 mma32c(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32c(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


constexpr float kNegBig = -1e30f;
constexpr float kLazy = 8.0f;   // log2 headroom before the reference max must move
constexpr float kSumBound = 4096.0f;   // a lane's tile sum past this: the tile's max is taken

// sum of the eight values plus c, fp32 accumulation (packed dot instructions against ones)
__device__ __forceinline__ float dot8_ones(const f16x8& a, float c) {
  typedef f16 h2 __attribute__((ext_vector_type(2)));
  const h2 one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_fdot2(h2{a[2 * i], a[2 * i + 1]}, one, c, false);
  return c;
}
__device__ __forceinline__ float dot8_ones(const bf16x8& a, float c) {
  typedef bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_fdot2_f32_bf16(b2{a[2 * i], a[2 * i + 1]}, one, c, false);
  return c;
}
constexpr int kKeysPerTile = 64;   // 128 halves the waits per key but leaves 2 instead of 3 workgroups per CU (slower)

// LDS rows of 128 bytes (8 chunks of 16): chunk c of row r sits in slot c ^ ((r >> 1) & 7), so any
// 16 consecutive rows read at one chunk cover all 64 banks.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
// K rows of KCH chunks: 4 or 8 chunks (64- or 128-byte rows) take swz8 modulo KCH; 256-byte rows
// (16 chunks) start on the same bank, so chunk c of row r sits in slot c ^ (r & 15)
template <int KCH>
__device__ __forceinline__ int kswz(int r) { return KCH >= 16 ? (r & 15) : swz8(r) % KCH; }
// Key order inside a 32-key S^T tile: the A operand row m holds key perm(m) (bits 2 and 3 swapped),
// which puts the 8 probabilities a lane feeds to one P.V step on 8 consecutive keys.
__device__ __forceinline__ int perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <typename T, int DQK, int DV, int KT>
__global__ __launch_bounds__(256, 2) void attn_time2_kernel(AttnLaunch L) {
  static_assert(KT % 32 == 0, "keys per tile");
  constexpr int RT = KT / 32;                // 32-key row tiles of S^T per key tile
  constexpr int KROWB = DQK * 2;             // bytes per K row
  constexpr int KCH = KROWB / 16;            // 16-byte chunks per K row
  constexpr int VROWB = KT * 2;              // bytes per V^T row (KT keys)
  constexpr int VCH = VROWB / 16;            // 16-byte chunks per V^T row
  constexpr int KBYTES = KT * KROWB, VBYTES = DV * VROWB;
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int KLD = KBYTES / (256 * 16), VLD = VBYTES / (256 * 16);   // loads per thread per stage
  constexpr int KSTEPS = DQK / 16;           // 32x32x16 steps over the q / k width for S
  constexpr int DT = DV / 32;                // 32-row d tiles of O^T
  static_assert(KLD >= 1 && VLD >= 1, "tile loader");
  using frag = typename Frag<T>::type;
  typedef typename Frag<T>::half_type h4;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  // workgroup order: all query blocks of one (seq, head) on one XCD
  const int nqb = L.npad / 128;
  const int nb = gridDim.x, per = nb >> 3, rem = nb & 7;
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int logical = x * per + min(x, rem) + slot;
  const int qb = logical % nqb, sh = logical / nqb;
  const int seq = sh / L.heads, h = sh - seq * L.heads;
  const int n = L.n, npad = L.npad;
  const int q0 = qb * 128 + w * 32;
  const size_t base = (size_t)sh * (size_t)npad * DQK, vbase = (size_t)sh * (size_t)npad * DV;
  const char* Qg = (const char*)((const T*)L.q + base);
  const char* Kg = (const char*)((const T*)L.k + base);
  const char* Vg = (const char*)((const T*)L.v + vbase);    // V^T [DV][npad]

  // this thread's DMA chunks: K slot c -> key c / KCH, physical chunk c % KCH holds logical chunk
  // (c % KCH) ^ (key % KCH); V^T slot c -> dim c / 8, 8 keys per chunk, same permutation by dim
  // K [npad][DH] and V^T [DH][npad] of this (sequence, head) as buffers
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kg, (uint32_t)(npad * DQK * 2));
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(Vg, (uint32_t)(npad * DV * 2));
  int ksrc[KLD], kdst[KLD];
#pragma unroll
  for (int j = 0; j < KLD; ++j) {
    const int c = j * 256 + threadIdx.x;
    const int row = c / KCH, pc = c % KCH;
    ksrc[j] = row * KROWB + ((pc ^ kswz<KCH>(row)) << 4);
    kdst[j] = (j * 256 + w * 64) * 16;
  }
  int vsrc[VLD], vdst[VLD];
#pragma unroll
  for (int j = 0; j < VLD; ++j) {
    const int c = j * 256 + threadIdx.x;
    const int row = c / VCH, pc = c % VCH;
    vsrc[j] = row * npad * 2 + ((pc ^ swz8(row)) << 4);
    vdst[j] = KBYTES + (j * 256 + w * 64) * 16;
  }
  auto issue = [&](int kt) {
    char* st = lds + (kt & 1) * STAGE;
#pragma unroll
    for (int j = 0; j < KLD; ++j) buffer_dma16(krs, ksrc[j], kt * KT * KROWB, st + kdst[j]);
#pragma unroll
    for (int j = 0; j < VLD; ++j) buffer_dma16(vrs, vsrc[j], kt * KT * 2, st + vdst[j]);
  };

  // the lane's gate, requested first (read at the end it would wait a memory round trip there)
  const float gate = q0 + l32 < n ? (L.gates ? L.gates[((size_t)seq * L.frames + q0 + l32) * L.heads + h] : 1.f) : 0.f;
  // q fragments: B operand of S^T = K Q^T; lane holds query q0 + l32, dims 16*ks + 8*g .. +7
  frag qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *(const frag*)(Qg + ((size_t)(q0 + l32) * DQK + 16 * ks + 8 * g) * 2);
  if (L.q_mul != 0.0f) {   // q not yet in log2 units: scaled once here, rounded to T
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = cvt<T>(tof<T>(qf[ks][e]) * L.q_mul);
  }

  f32x16 o[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[d][v] = 0.f;
  // q arrives scaled by log2(e) (and 1/sqrt(dh)), so scores are already in log2 units; the S^T
  // accumulators start at -mref, so the products deliver s - mref and p = exp2 of it directly
  float mref = 0.f;
  float lsum_p = 0.f;   // the lane's part of its query's row sum (16 of every 32 keys)
  f32x16 negm;   // -mref in every element: the C operand of each tile's first S^T step
#pragma unroll
  for (int v = 0; v < 16; ++v) negm[v] = 0.f;

  const int ntiles = (n + KT - 1) / KT;
  issue(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    if (kt + 1 < ntiles) issue(kt + 1);
    const char* st = lds + (kt & 1) * STAGE;

    f32x16 s[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = r * 32 + perm(l32);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int lc = 2 * ks + g;
        const frag a = *(const frag*)(st + row * KROWB + ((lc ^ kswz<KCH>(row)) << 4));
        if (ks == 0) s[r] = mma32c(a, qf[0], negm);
        else mma32(s[r], a, qf[ks]);
      }
    }
    if (kt == ntiles - 1 && (n & (KT - 1))) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt * KT + r * 32 + perm(8 * (v >> 2) + 4 * g + (v & 3));
          if (key >= n) s[r][v] = kNegBig;
        }
    }
    // probabilities against the current reference, rounded to T, and the lane's sum of the rounded
    // values (the ones the P.V product uses; packed dot instructions against ones)
    frag pf[2 * RT];
    auto probs = [&]() -> float {
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 2 * RT; ++t) {
        const int r = t >> 1, hv = (t & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[t][e] = cvt<T>(__builtin_amdgcn_exp2f(s[r][hv + e]));
        sum = dot8_ones(pf[t], sum);
      }
      return sum;
    };
    // tile 0 sets the reference to its max; a later tile keeps it unless a lane's sum passes
    // kSumBound (then some probability passed kSumBound / 32): only then is the tile's max taken
    // and the reference moved as below
    float tsum = 0.f;
    bool redo = kt == 0;
    if (!redo) {
      tsum = probs();
      redo = __any(!(tsum <= kSumBound));
    }
    if (redo) {
      float mx = kNegBig;
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[r][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // the first tile sets the reference exactly; later ones move it only past kLazy
      if (kt == 0 || __any(mx > kLazy)) {
        const float up = kt == 0 ? mx : fmaxf(mx, 0.f);
        if (kt > 0) {
          const float alpha = __builtin_amdgcn_exp2f(-up);
#pragma unroll
          for (int d = 0; d < DT; ++d) o[d] *= alpha;
          lsum_p *= alpha;
        }
        mref += up;
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[v] = -mref;
#pragma unroll
        for (int r = 0; r < RT; ++r) s[r] -= up;
      }
      tsum = probs();
    }
    lsum_p += tsum;
#pragma unroll
    for (int t = 0; t < 2 * RT; ++t) {
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        // V^T row (head dim) d*32 + l32, keys 16t + 8g .. +7: one 16-byte chunk
        const int row = d * 32 + l32;
        const frag a = *(const frag*)(st + KBYTES + row * VROWB + (((2 * t + g) ^ swz8(row)) << 4));
        mma32(o[d], a, pf[t]);
      }
    }
  }

  const float lsum = lsum_p + __shfl_xor(lsum_p, 32, 64);   // lanes l and l ^ 32 hold one query
  const int q = q0 + l32;
  if (q >= n) return;
  const size_t row = (size_t)seq * L.frames + q;
  const float scale = gate / lsum;
  T* dst = (T*)L.o + row * (L.heads * DV) + h * DV;
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      h4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = cvt<T>(o[d][4 * b4 + e] * scale);
      *(h4*)(dst + d * 32 + 8 * b4 + 4 * g) = out;
    }
}

template <typename T>
hipError_t launch_t(const AttnLaunch& L, hipStream_t stream) {
  dim3 grid((L.npad / 128) * L.heads * L.seqs), block(256);
  const int dv = L.dv ? L.dv : L.dh;
  if (L.dh == 64 && dv == 64) hipLaunchKernelGGL((attn_time2_kernel<T, 64, 64, kKeysPerTile>), grid, block, 0, stream, L);
  else if (L.dh == 32 && dv == 32) hipLaunchKernelGGL((attn_time2_kernel<T, 32, 32, kKeysPerTile>), grid, block, 0, stream, L);
  else if (L.dh == 128 && dv == 64) hipLaunchKernelGGL((attn_time2_kernel<T, 128, 64, kKeysPerTile>), grid, block, 0, stream, L);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool attention_time2_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 32 && dv == 32) || (dqk == 128 && dv == 64);
}

hipError_t launch_attention_time2(const AttnLaunch& L, hipStream_t stream) {
  // q must carry log2(e) (and the score scale), or q_mul must bring it
  if (L.npad % 128 || L.npad < L.n || L.n < 1 || L.axis != 0 || L.scale_log2 != 1.0f) return hipErrorInvalidValue;
  if (!attention_time2_supported(L.dh, L.dv ? L.dv : L.dh)) return hipErrorInvalidValue;
  switch (L.dtype) {
    case DT_F16: return launch_t<f16>(L, stream);
    case DT_BF16: return launch_t<bf16>(L, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mbr
