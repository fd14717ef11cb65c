// MFMA GEMM for 16-bit operands (fp16 / bf16) on gfx950: C = A . B^T with fused epilogues.
//
// Same problems and epilogues as the generic family (k_gemm.hip) — the linear layers of the core
// ([P1] "Per Attention layer", "Parameter accounting"; [P5] export-roformer.py classes Attn, FF and
// the mask MLP) — laid out for the CDNA4 matrix cores:
//   * block tile BM x BN over a WM x WN grid of waves; every wave owns (BM/WM) x 64 of C as 32 x 32
//     tiles on v_mfma_f32_32x32x16 (each lane feeds 16 bytes of A and of B per 32 x 32 x 16 product);
//   * K in steps of 32 elements (64-byte rows) through an NS-stage LDS ring filled by 16-byte direct
//     global->LDS loads, NS-1 stages in flight while one is consumed; each wave waits for its own
//     loads with s_waitcnt and the workgroup meets at one barrier per step;
//   * rows are stored with their four 16-byte chunks XOR-permuted by ((row>>1) ^ (row>>2)) & 3 so
//     the 32 rows one fragment read touches fall on distinct LDS banks;
//   * launches walk the tiles (dense order, or the grouped launch's tile table, where a group's
//     tiles are consecutive) so that each XCD (workgroups are dealt round-robin to the 8 XCDs)
//     receives one contiguous run of tiles: neighbouring tiles share operand panels in that XCD's
//     L2;
//   * each tile walks K starting at chunk (column tile mod K/32), so the tiles reading one A panel
//     at the same time ask for different chunks and the later ones hit L2;
//   * the epilogue stages 32 accumulator rows of a wave at a time through LDS and writes 16-byte
//     vectors: rows of q, k, v (rotary applied to the pairs a lane already holds; the time axis'
//     v transposed, 8 bytes of 4 positions per lane), GELU / tanh outputs, fp32 residual updates,
//     and the GLU of paired 32-feature value / gate blocks stored feature-major.
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

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }


// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima), plus a compiler barrier.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <typename T> struct Pack8;
template <> struct Pack8<f16> { typedef f16x8 type; };
template <> struct Pack8<bf16> { typedef bf16x8 type; };

template <int BM_, int WM_, int WN_, int NS_>
struct Cfg {
  static constexpr int BM = BM_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int BN = 64 * WN;                 // every wave owns 64 columns
  static constexpr int WROWS = BM / WM;              // rows per wave (64 or 128)
  static constexpr int TM = WROWS / 32;              // 32 x 32 tiles per wave along M
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int ROWB = 64;                    // bytes per LDS row and stage (32 elements)
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LD = BM * 4 / THREADS, B_LD = BN * 4 / THREADS;
  static constexpr int LOADS = A_LD + B_LD;
  static constexpr int EP_STRIDE = 68;              // floats per staged row (64 + 4)
  static constexpr int EP_WAVE = 32 * EP_STRIDE * 4;
  static constexpr int LDS = (NS * STAGE > WM * WN * EP_WAVE) ? NS * STAGE : WM * WN * EP_WAVE;
  static_assert(A_LD * THREADS == BM * 4 && B_LD * THREADS == BN * 4, "whole loads per thread");
  static_assert(WROWS % 32 == 0, "wave rows");
  static_assert(LOADS * (NS - 2) < 64, "vmcnt range");
};

template <typename T, int EPI, class C>
__global__ __launch_bounds__(C::THREADS) void gemm2_kernel(GemmLaunch L) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using frag = typename Frag<T>::type;
  constexpr int BM = C::BM, BN = C::BN, NS = C::NS, ROWB = C::ROWB, TM = C::TM;
  constexpr int NW = C::WM * C::WN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / C::WN, wn = w % C::WN;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // wave-uniform: LDS targets stay scalar
  const int M = L.M;
  GemmGroup g;
  int m0, n0;
  // workgroups are dealt round-robin to the 8 XCDs: walk the tiles so that each XCD gets one
  // contiguous run of them (neighbouring tiles share operand panels in that XCD's L2)
  const int nb = gridDim.x, per = nb >> 3, rem = nb & 7;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int logical = xcd * per + min(xcd, rem) + slot;
  if (L.tiles) {
    const GemmTile t = L.tiles[logical];
    g = L.groups[t.group];
    m0 = t.m0;
    n0 = t.n0;
  } else {
    g = L.dense;
    const int tn = (g.N + BN - 1) / BN;
    m0 = (logical / tn) * BM;
    n0 = (logical % tn) * BN;
  }
  if (m0 >= M) return;

  // ---- loader: this thread's 16-byte chunks of a stage, from buffers over this tile's A rows
  // and B rows (rows past the end read the last row), into wave-uniform LDS targets
  const int64_t lda_b = (int64_t)g.lda * 2, ldb_b = (int64_t)g.ldb * 2;
  const int arows = min(BM, M - m0), brows = max(1, min(BN, g.N - n0));
  const __amdgpu_buffer_rsrc_t ars = buffer_rsrc_uniform(
      (const char*)L.A + (g.a_off0 + g.a_offb * (int64_t)M) * 2 + (int64_t)m0 * lda_b, (uint32_t)(arows * lda_b));
  const __amdgpu_buffer_rsrc_t brs =
      buffer_rsrc_uniform((const char*)L.B + g.b_off * 2 + (int64_t)n0 * ldb_b, (uint32_t)(brows * ldb_b));
  int voff[C::LOADS], dst[C::LOADS];
#pragma unroll
  for (int j = 0; j < C::A_LD; ++j) {
    const int row = (j * NW + w) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    voff[j] = (int)(min(row, arows - 1) * lda_b) + c * 16;
    dst[j] = (j * NW + wu) * 1024;
  }
#pragma unroll
  for (int j = 0; j < C::B_LD; ++j) {
    const int row = (j * NW + w) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    voff[C::A_LD + j] = (int)(min(row, brows - 1) * ldb_b) + c * 16;
    dst[C::A_LD + j] = C::A_BYTES + (j * NW + wu) * 1024;
  }
  // K order rotated by the column tile: the tiles that share an A panel (same m0) run at the same
  // time, and in plain order all of them would ask for each K chunk at once and every one would
  // wait for the same HBM fill.  Rotated by one chunk per column tile, their prologues request the
  // whole panel together and the later steps find their chunk already in L2.  (Only the column
  // tile: a row's sum order must not depend on where the row sits in the batch.)
  const int nk = g.K >> 5;
  const int krot = nk > 1 ? (n0 / BN) % nk : 0;
  auto issue = [&](int ks) {
    char* base = smem + (ks % NS) * C::STAGE;
    int kc = ks + krot;
    if (kc >= nk) kc -= nk;
    const int ko = kc * 64;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) buffer_dma16(j < C::A_LD ? ars : brs, voff[j], ko, base + dst[j]);
  };

  f32x16 acc[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);
  const int r32 = lane & 31, khalf = lane >> 5;
  // fragment row offsets and their chunk permutations (loop invariant)
  int arow[TM], aswz[TM], brow[2], bswz[2];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = wm * C::WROWS + i * 32 + r32;
    arow[i] = row * ROWB;
    aswz[i] = swz(row);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = wn * 64 + j * 32 + r32;
    brow[j] = C::A_BYTES + row * ROWB;
    bswz[j] = swz(row);
  }
  for (int kk = 0; kk < nk; ++kk) {
    // stages issued so far: min(nk, kk + NS - 1); stage kk must be complete
    const int ahead = min(nk - 1 - kk, NS - 2);
    if (ahead >= NS - 2) {
      wait_vm<C::LOADS * (NS - 2)>();
    } else if constexpr (NS > 3) {
      if (ahead == 1) wait_vm<C::LOADS>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    block_barrier();
    const char* st = smem + (kk % NS) * C::STAGE;
    // all fragment reads of the step first, then the products: the first products wait only for
    // their own operands while the later reads are still in flight
    frag a[2][TM], b[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 2 * ks + khalf;
#pragma unroll
      for (int i = 0; i < TM; ++i) a[ks][i] = *(const frag*)(st + arow[i] + ((c ^ aswz[i]) << 4));
#pragma unroll
      for (int j = 0; j < 2; ++j) b[ks][j] = *(const frag*)(st + brow[j] + ((c ^ bswz[j]) << 4));
    }
    if (kk + NS - 1 < nk) issue(kk + NS - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma32(acc[i][j], a[ks][i], b[ks][j]);
  }

  // ---- epilogue: every wave is done with the ring once all have passed this barrier
  block_barrier();
  const int cbase = n0 + wn * 64;
  if (cbase >= g.N) return;
  float* ep = (float*)(smem + w * C::EP_WAVE);
  const float* bias = L.bias ? L.bias + g.bias_off : nullptr;
  constexpr int ES = C::EP_STRIDE;
  // global row of a local row (grouped EMBED / TANH launches: group e0's rows start at e0 * M)
  const int64_t grow0 = (L.tiles && (EPI == EPI_EMBED || EPI == EPI_TANH)) ? (int64_t)g.e0 * M : 0;
  // sum of a row's partial sums of squares (kSsStride slots, the unused ones stay zero): four
  // independent 16-byte loads
  auto row_ss = [&](const float* base, int64_t grow) -> float {
    const float4* p = (const float4*)(base + grow * kSsStride);
    const float4 a = p[0], b = p[1], c = p[2], d = p[3];
    return ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w)) + ((c.x + c.y) + (c.z + c.w)) +
           ((d.x + d.y) + (d.z + d.w));
  };
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    // stage rows i*32 .. i*32+31 of this wave's tile
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) ep[(8 * (v >> 2) + 4 * khalf + (v & 3)) * ES + j * 32 + r32] = acc[i][j][v];
    const int rbase = m0 + wm * C::WROWS + i * 32;
    // per-row factors of this pass, computed once by lane r%32 for row rbase + r%32 and read by
    // the lanes that need them through a shuffle: the consumer row scale, and the producer-side
    // normalisation of the residual read
    float sc_mine = 1.0f, si_mine = 1.0f;
    {
      const int myrow = rbase + r32;
      if (myrow < M) {
        if (L.rowss) sc_mine = L.rs_mul / fmaxf(sqrtf(row_ss(L.rowss, grow0 + myrow)), kNormEps);
        if (L.in_ss) si_mine = 1.0f / fmaxf(sqrtf(row_ss(L.in_ss, grow0 + myrow)), kNormEps);
      }
    }
    if constexpr (EPI == EPI_RESID || EPI == EPI_FFN2 || EPI == EPI_EMBED) {
      // fp32 rows of 64 columns: 16 lanes x 4 floats per row, 4 rows per pass
      const int c4 = (lane & 15) * 4;
      float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bias) bv = *(const float4*)(bias + cbase + c4);
      float4 ing = make_float4(1.f, 1.f, 1.f, 1.f), xg = make_float4(1.f, 1.f, 1.f, 1.f);
      if (L.in_gain) ing = *(const float4*)(L.in_gain + cbase + c4);
      if (L.xh_gain) {
        const float4 t4 = *(const float4*)(L.xh_gain + cbase + c4);
        xg = make_float4(t4.x * L.xh_gmul, t4.y * L.xh_gmul, t4.z * L.xh_gmul, t4.w * L.xh_gmul);
      }
      float* Cp = (float*)L.C + g.c_off0 + g.c_offb * (int64_t)M;
#pragma unroll 2
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int row = rbase + r;
        const bool active = row < M;           // uniform over the 16 lanes of a row
        const float4 a = *(const float4*)(ep + r * ES + c4);
        float4* o = (float4*)(Cp + (int64_t)row * L.ldc + cbase + c4);
        float4 val = make_float4(a.x + bv.x, a.y + bv.y, a.z + bv.z, a.w + bv.w);
        const float si = __shfl(si_mine, r, 64);
        if constexpr (EPI == EPI_RESID || EPI == EPI_FFN2) {
          float4 xo = active ? *o : make_float4(0.f, 0.f, 0.f, 0.f);
          if (L.in_ss) xo = make_float4(xo.x * ing.x * si, xo.y * ing.y * si, xo.z * ing.z * si, xo.w * ing.w * si);
          val = make_float4(xo.x + val.x, xo.y + val.y, xo.z + val.z, xo.w + val.w);
        }
        if (active) *o = val;
        const float4 hv = make_float4(val.x * xg.x, val.y * xg.y, val.z * xg.z, val.w * xg.w);
        if (L.xh && active) {
          typename Vec4<T>::type h4;
          h4[0] = cvt<T>(hv.x); h4[1] = cvt<T>(hv.y); h4[2] = cvt<T>(hv.z); h4[3] = cvt<T>(hv.w);
          *(typename Vec4<T>::type*)((T*)L.xh + (grow0 + row) * L.ldc + cbase + c4) = h4;
        }
        if (L.ss1) {
          float q1 = val.x * val.x + val.y * val.y + val.z * val.z + val.w * val.w;
          q1 += __shfl_xor(q1, 8, 64);
          q1 += __shfl_xor(q1, 4, 64);
          q1 += __shfl_xor(q1, 2, 64);
          q1 += __shfl_xor(q1, 1, 64);
          if (active && (lane & 15) == 0) L.ss1[(grow0 + row) * kSsStride + (cbase >> 6)] = q1;
        }
        if (L.ss2) {
          float q2 = hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w;
          q2 += __shfl_xor(q2, 8, 64);
          q2 += __shfl_xor(q2, 4, 64);
          q2 += __shfl_xor(q2, 2, 64);
          q2 += __shfl_xor(q2, 1, 64);
          if (active && (lane & 15) == 0) L.ss2[(grow0 + row) * kSsStride + (cbase >> 6)] = q2;
        }
      }
    } else if constexpr (EPI == EPI_GLU) {
      // 32 value columns then their 32 gate columns; lane%32 = row, lane/32 picks 16 features
      float* out = (float*)L.C + g.c_off0 + g.c_offb * (int64_t)M;
      const int row = rbase + r32;
      const int T_ = L.glu_frames;
      const int b = row / T_, t = row - b * T_;
      const int f0 = (cbase >> 6) * 32 + khalf * 16;
#pragma unroll 4
      for (int e = 0; e < 16; ++e) {
        const int col = khalf * 16 + e;
        if (f0 + e >= g.e1) break;
        const float val = (ep[r32 * ES + col] + bias[cbase + col]) *
                          sigmoidf_(ep[r32 * ES + 32 + col] + bias[cbase + 32 + col]);
        if (row < M) out[((int64_t)b * L.glu_total + g.e0 + f0 + e) * T_ + t] = val;
      }
    } else {
      typedef typename Pack8<T>::type pack;
      const QkvArgs& qa = L.qkv;
      int which = 0;
      if constexpr (EPI == EPI_QKV) which = cbase / (qa.heads * qa.dh);
      if (EPI == EPI_QKV && which == 2 && qa.axis == 0) {
        // time axis: v goes out transposed, [seq][h][dh][npad]
        const int seq0 = rbase / qa.frames, pos0 = rbase - seq0 * qa.frames;
        if (rbase + 32 <= M && pos0 + 32 <= qa.frames && (pos0 & 3) == 0) {
          // the 32 rows are positions pos0 .. pos0+31 of one sequence, pos0 a multiple of 4: lane
          // (column 8k + lane/8, rows 4(lane%8) .. +3) writes 8 bytes, so 8 lanes fill 64 bytes of
          // one V^T row and an instruction covers 8 of them
          const int j = lane & 7;
          float scr[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) scr[t] = __shfl(sc_mine, 4 * j + t, 64);
          T* vt = (T*)qa.v + ((size_t)seq0 * qa.heads * qa.dh + (cbase - 2 * qa.heads * qa.dh)) * qa.npad + pos0 + 4 * j;
#pragma unroll 4
          for (int k = 0; k < 8; ++k) {
            const int c = 8 * k + (lane >> 3);
            typename Vec4<T>::type h4;
#pragma unroll
            for (int t = 0; t < 4; ++t) h4[t] = cvt<T>(ep[(4 * j + t) * ES + c] * scr[t]);
            *(typename Vec4<T>::type*)(vt + (size_t)c * qa.npad) = h4;
          }
          continue;
        }
        // otherwise lane%32 = row: every store instruction writes 32 consecutive positions of one
        // head dimension per half wave
        const int row = rbase + r32;
        if (row < M) {
          const float sc = sc_mine;
          const int seq = row / qa.frames, pos = row - seq * qa.frames;
          T* vt = (T*)qa.v + (size_t)seq * qa.heads * qa.dh * qa.npad + pos;
          const int f0 = cbase - 2 * qa.heads * qa.dh + khalf * 32;  // v feature h*dh + d
#pragma unroll 8
          for (int d = 0; d < 32; ++d) vt[(size_t)(f0 + d) * qa.npad] = cvt<T>(ep[r32 * ES + khalf * 32 + d] * sc);
        }
        continue;
      }
      // 16-bit rows of 64 columns: 8 lanes x 8 elements per row, 8 rows per pass
      const int c8 = (lane & 7) * 8;
      int h = 0, d0 = 0;
      if constexpr (EPI == EPI_QKV) {
        if (which < 3) {
          const int f = cbase + c8 - which * qa.heads * qa.dh;
          h = f / qa.dh;
          d0 = f - h * qa.dh;
        }
      }
      float bvals[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bvals[e] = bias ? bias[cbase + c8 + e] : 0.f;
      // sequence / position of this lane's first row; later rows step by 8 (at most one wrap
      // per step when a sequence is at least 8 long, loops otherwise)
      int seqs[4] = {0, 0, 0, 0}, poss[4] = {0, 0, 0, 0};
      float4 csv[4], snv[4];
      if constexpr (EPI == EPI_QKV) {
        int seq, pos, wrap;
        const int r0 = rbase + (lane >> 3);
        if (qa.axis == 0) {
          wrap = qa.frames;
          seq = r0 / wrap;
          pos = r0 - seq * wrap;
        } else {
          wrap = qa.batch * qa.frames;
          pos = r0 / wrap;
          seq = r0 - pos * wrap;
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          if (it > 0) {
            // advance the (seq, pos) pair by 8 rows
            if (qa.axis == 0) {
              pos += 8;
              while (pos >= wrap) { pos -= wrap; ++seq; }
            } else {
              seq += 8;
              while (seq >= wrap) { seq -= wrap; ++pos; }
            }
          }
          seqs[it] = seq;
          poss[it] = pos;
        }
        // the rotary factors of the four rows, all loaded before the first is used
        if (which < 2)
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int pr = rbase + it * 8 + (lane >> 3) < M ? poss[it] : 0;
            csv[it] = *(const float4*)(qa.cos + pr * (qa.dh >> 1) + (d0 >> 1));
            snv[it] = *(const float4*)(qa.sin + pr * (qa.dh >> 1) + (d0 >> 1));
          }
      }
      constexpr int kRowUnroll = EPI == EPI_QKV ? 4 : 2;   // QKV: its per-row arrays stay in registers
#pragma unroll kRowUnroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int row = rbase + r;
        const float sc = __shfl(sc_mine, r, 64);
        const int seq = seqs[it], pos = poss[it];
        if (row >= M) continue;
        const float4 a0 = *(const float4*)(ep + r * ES + c8);
        const float4 a1 = *(const float4*)(ep + r * ES + c8 + 4);
        float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        if (L.rowss) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= sc;
        }
        pack p;
        if constexpr (EPI == EPI_QKV) {
          if (which == 3) {
            // attention gates: one per head, sigmoid of the normalised row's projection + bias
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int hh = c8 + e;
              if (hh < qa.heads) L.gates[(size_t)row * qa.heads + hh] = sigmoidf_(v[e] + L.gate_bias[hh]);
            }
            continue;
          }
          if (which < 2) {
            const float4 cs = csv[it], sn = snv[it];
            const float cc[4] = {cs.x, cs.y, cs.z, cs.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x0 = v[2 * q], x1 = v[2 * q + 1];
              v[2 * q] = x0 * cc[q] - x1 * ss[q];
              v[2 * q + 1] = x0 * ss[q] + x1 * cc[q];
            }
            if (which == 0) {
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] *= qa.q_mul;
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = cvt<T>(v[e]);
          T* dstp = (T*)(which == 0 ? qa.q : which == 1 ? qa.k : qa.v);
          *(pack*)(dstp + (((size_t)seq * qa.heads + h) * qa.npad + pos) * qa.dh + d0) = p;
        } else {
          T* Cp = (T*)L.C + g.c_off0 + g.c_offb * (int64_t)M;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xv = v[e] + bvals[e];
            if constexpr (EPI == EPI_GELU) p[e] = cvt<T>(0.5f * gelu2_tail(xv));   // rounded to 16 bits
            else if constexpr (EPI == EPI_TANH) p[e] = cvt<T>(tanh_fast(xv));
            else p[e] = cvt<T>(xv);
          }
          *(pack*)(Cp + (int64_t)row * L.ldc + cbase + c8) = p;
        }
      }
    }
  }
}

// Tile configurations (index = variant):
//   0: 256 x 128, 2 x 2 waves of 128 x 64, 3 stages      3: 128 x 256, 2 x 4 waves of 64 x 64, 4 stages
//   1: 128 x 128, 2 x 2 waves of  64 x 64, 4 stages      4: 256 x 128, 4 x 2 waves of 64 x 64, 3 stages
//   2: 256 x 256, 2 x 4 waves of 128 x 64, 3 stages      5: 128 x 128, 2 x 2 waves of 64 x 64, 3 stages
typedef Cfg<256, 2, 2, 3> C0;
typedef Cfg<128, 2, 2, 4> C1;
typedef Cfg<256, 2, 4, 3> C2;
typedef Cfg<128, 2, 4, 4> C3;
typedef Cfg<256, 4, 2, 3> C4;
typedef Cfg<128, 2, 2, 3> C5;

template <typename T, int EPI, class C>
hipError_t launch_cfg(const GemmLaunch& L, hipStream_t stream) {
  int blocks;
  if (L.tiles) {
    blocks = L.n_tiles;
  } else {
    if (L.dense.N % 64 || L.dense.K % 32) return hipErrorInvalidValue;
    blocks = ((L.M + C::BM - 1) / C::BM) * ((L.dense.N + C::BN - 1) / C::BN);
  }
  if (blocks <= 0) return hipSuccess;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm2_kernel<T, EPI, C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((gemm2_kernel<T, EPI, C>), dim3(blocks), dim3(C::THREADS), C::LDS, stream, L);
  return hipGetLastError();
}

template <typename T, int EPI>
hipError_t launch_epi(const GemmLaunch& L, int variant, hipStream_t stream) {
  switch (variant) {
    case 0: return launch_cfg<T, EPI, C0>(L, stream);
    case 1: return launch_cfg<T, EPI, C1>(L, stream);
    case 2: return launch_cfg<T, EPI, C2>(L, stream);
    case 3: return launch_cfg<T, EPI, C3>(L, stream);
    case 4: return launch_cfg<T, EPI, C4>(L, stream);
    case 5: return launch_cfg<T, EPI, C5>(L, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_t(const GemmLaunch& L, int variant, hipStream_t stream) {
  switch (L.epi) {
    case EPI_EMBED: return launch_epi<T, EPI_EMBED>(L, variant, stream);
    case EPI_QKV: return launch_epi<T, EPI_QKV>(L, variant, stream);
    case EPI_GELU: return launch_epi<T, EPI_GELU>(L, variant, stream);
    case EPI_RESID: return launch_epi<T, EPI_RESID>(L, variant, stream);
    case EPI_TANH: return launch_epi<T, EPI_TANH>(L, variant, stream);
    case EPI_GLU: return launch_epi<T, EPI_GLU>(L, variant, stream);
    case EPI_STORE16: return launch_epi<T, EPI_STORE16>(L, variant, stream);
    case EPI_FFN2: return launch_epi<T, EPI_FFN2>(L, variant, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemm2_variants() { return 6; }
int gemm2_tile_rows(int variant) {
  switch (variant) {
    case 0: return C0::BM;
    case 1: return C1::BM;
    case 2: return C2::BM;
    case 3: return C3::BM;
    case 4: return C4::BM;
    case 5: return C5::BM;
  }
  return -1;
}
int gemm2_tile_cols(int variant) {
  switch (variant) {
    case 0: return C0::BN;
    case 1: return C1::BN;
    case 2: return C2::BN;
    case 3: return C3::BN;
    case 4: return C4::BN;
    case 5: return C5::BN;
  }
  return -1;
}

hipError_t launch_gemm2(const GemmLaunch& L, int variant, hipStream_t stream) {
  switch (L.dtype) {
    case DT_F16: return launch_t<f16>(L, variant, stream);
    case DT_BF16: return launch_t<bf16>(L, variant, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mbr
