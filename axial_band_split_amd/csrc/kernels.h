// Launchers of the core's HIP kernels (host side) and the descriptors they share with the
// library.  Every launcher enqueues on `stream` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mbr {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// One problem of a grouped GEMM  C = A . B^T  (A [M, K] row-major, B [N, K] row-major: the
// weights in their [out, in] form).  Offsets are in elements; the parts marked "b" are multiplied
// by the forward's rows per group (batch * frames) at run time, so one descriptor serves every
// batch size.
struct GemmGroup {
  int64_t a_off0, a_offb;   // A element offset = a_off0 + a_offb * rows
  int64_t b_off;            // B element offset
  int64_t c_off0, c_offb;   // C element offset (epilogue-specific meaning)
  int64_t bias_off;         // bias element offset
  int32_t N, K, lda, ldb;
  int32_t e0, e1;           // epilogue extras (GLU: feature offset, band width)
};

constexpr int kSsStride = 16;   // floats per row of the row-statistics buffers (D <= 1024)

struct GemmTile {
  int32_t group, m0, n0, pad;
};

// Epilogue kinds of the GEMM family.
enum Epi {
  EPI_EMBED = 0,     // C(float) = acc + bias                      (band embedding)
  EPI_QKV = 1,       // rotary on q, k; scatter q, k, v^T into attention layout
  EPI_GELU = 2,      // C(T) = gelu(acc + bias)                       (FFN1)
  EPI_RESID = 3,     // C(float) += acc (+ bias)                      (out-proj, FFN2)
  EPI_TANH = 4,      // C(T) = tanh(acc + bias)                       (mask MLP hidden layers)
  EPI_GLU = 5,       // paired value/gate column blocks -> value*sigmoid(gate), feature-major float
  EPI_STORE16 = 6,   // C(T) = acc + bias                             (16-bit kernel; test surface)
  EPI_FFN2 = 7,      // as EPI_RESID, for the feed-forward's second layer (its own kernel name)
};

struct QkvArgs {
  void* q;            // [seqs][H][npad][dh]
  void* k;            // [seqs][H][npad][dh]
  void* v;            // [seqs][H][npad][dh]
  const float* cos;   // [npos][dh/2]
  const float* sin;
  int32_t axis;       // 0: time (seq = row / T, pos = row % T); 1: band (seq = row % (B*T), pos = row / (B*T))
  int32_t frames, batch, heads, dh, npad;
  float q_mul;        // factor on q after the rotary step (16-bit path: log2(e), scores in log2 units)
};

struct GemmLaunch {
  int dtype;                    // DT_*
  int epi;                      // Epi
  const void* A;
  const void* B;
  void* C;
  const float* bias;
  int64_t ldc;
  int32_t M;                    // rows of every group for this launch
  // dense (single-problem) launch when tiles == nullptr
  GemmGroup dense;
  // grouped launch
  const GemmGroup* groups;      // device array
  const GemmTile* tiles;        // device array
  int32_t n_tiles;
  QkvArgs qkv;
  // GLU output layout: C[(b)][feature][t] with total features `glu_total`, frames `glu_frames`
  int32_t glu_total, glu_frames;
  // ---- row statistics (16-bit kernel only).  Row partial sums of squares are kept per 64-column
  // block of a D-wide row: ss[row * kSsStride + column / 64] (slots past D/64 stay zero).  For
  // grouped launches (EMBED, TANH) the global row of a group's local row r is g.e0 * M + r.
  // consumer side: scale row r of the product by rs_mul / max(sqrt(sum of rowss[r][*]), 1e-12)
  const float* rowss;
  int32_t ss_parts;
  float rs_mul;
  // RESID: the residual read from C is first normalised: x * in_gain[col] / max(|x|, 1e-12)
  const float* in_ss;
  const float* in_gain;
  // RESID / EMBED producer side: xh[row][col] = T(x_new * xh_gain[col] * xh_gmul) (gain optional),
  // ss1 partials of x_new^2, ss2 partials of (x_new * xh_gain * xh_gmul)^2
  void* xh;
  const float* xh_gain;
  float xh_gmul;
  float* ss1;
  float* ss2;
  // QKV: columns 3*H*dh .. 3*H*dh + H - 1 are the attention gates: gates[row][h] = sigmoid(. + bias)
  float* gates;
  const float* gate_bias;
};

// Generic 128 x 128 tile kernel (every dtype; the fp32 path uses it).  GLU pairs 16-column blocks.
hipError_t launch_gemm(const GemmLaunch& L, hipStream_t stream);
// 16-bit operand kernel (fp16 / bf16) in several tile configurations (`variant`, see k_gemm2.hip);
// needs N % 64 == 0 and K % 32 == 0; grouped tile tables must use the variant's tile rows and
// columns.  GLU pairs 32-column blocks.
hipError_t launch_gemm2(const GemmLaunch& L, int variant, hipStream_t stream);
int gemm2_variants();
int gemm2_tile_rows(int variant);
int gemm2_tile_cols(int variant);

// Row RMS norm passes over the fp32 residual stream x [rows, D].
//   mode 0: xh = T(x * sqrt(D) / max(|x|, eps)); gates (optional) from the same normalised row
//   mode 1: y = x * gain / max(|x|, eps); x = y; then xh, gates as mode 0 applied to y
//   mode 2: y = x * gain / max(|x|, eps); x = y; xh = T(y)
struct NormLaunch {
  int dtype;
  int mode;
  float* x;
  void* xh;
  const float* gain;       // [D] (gamma * sqrt(D)) for modes 1, 2
  float* gates;            // [rows, H] or nullptr
  const float* wg;         // [H, D] gate weights (gamma folded), fp32
  const float* bg;         // [H]
  int32_t rows, D, H;
};
hipError_t launch_norm(const NormLaunch& L, hipStream_t stream);

// Band gather + per-band L2 normalisation of the complex stereo input into the half/float
// matrix U: per band i, rows b*T + t, columns = band features (zero padded to kpad_i).
struct GatherLaunch {
  int dtype;
  const float* in;
  void* U;
  const int32_t* band_info;   // [NB][4]: feature offset, width, kpad, U column offset (sum of kpad before)
  const int32_t* gather_pair; // slot -> pair
  int32_t num_bands, batch, frames, n_freqs, channels, layout, max_kpad;
};
hipError_t launch_gather(const GatherLaunch& L, hipStream_t stream);

// Band gather and band embedding in one kernel (k_embed.hip, 16-bit path): X = RMSNorm(gathered
// band) W_i^T + b_i in fp32, XH = the same in 16 bits, ss = its row sums of squares per 64 columns.
struct EmbedLaunch {
  int dtype;
  const float* in;            // the spectrum, io layout 0 or 1
  const void* W;              // band weights in fragment order (see embed_stream in mbr_core.cpp)
  const int32_t* w_off;       // [NB] element offset of band i's fragments from W
  const int32_t* order;       // [NB] band indices, widest first
  const int32_t* band_info;   // [NB][4] as for the gather
  const int32_t* gather_pair; // slot -> pair
  const float* bias;          // [NB][D]
  float* X;                   // [NB][batch * frames][D]
  void* XH;                   // same, 16-bit
  float* ss;                  // [NB * batch * frames][kSsStride]
  int32_t num_bands, batch, frames, n_freqs, channels, layout, D, max_kpad;
};
bool embed_fused_supported(int dtype, int D, int max_kpad);
hipError_t launch_embed(const EmbedLaunch& L, hipStream_t stream);

// Attention over sequences held in [seqs][H][npad][dh] (q, k, v);
// writes O * gate into token layout O[row][H*dh].
struct AttnLaunch {
  int dtype;
  int axis;                 // 0 time (flash, n = T), 1 band (n = NB <= 64, one wave per sequence-head)
  const void* q;
  const void* k;
  const void* v;
  const float* gates;       // [rows][H]
  void* o;                  // [rows][H*dh]
  int32_t n, npad, seqs, heads, dh, frames, batch;
  float scale_log2;         // dh^-1/2 * log2(e) when the scale is not folded; 1*log2(e) otherwise
  // 16-bit time kernel only: v width when it differs from the q / k width dh (0: dh), and a factor
  // applied to q as it is loaded (0: none, q arrives in log2 units with its scale, as the
  // projection writes it); gates may be NULL there (every gate 1)
  int32_t dv;
  float q_mul;
};
hipError_t launch_attention(const AttnLaunch& L, hipStream_t stream);
// Time axis, 16-bit operands: v must be V^T [seqs][H][dh][npad] (the 16-bit q/k/v projection writes
// it that way for the time axis); npad % 128 == 0.
hipError_t launch_attention_time2(const AttnLaunch& L, hipStream_t stream);
bool attention_time2_supported(int dqk, int dv);

// The band axis' q, k, v projection, rotary, attention over the bands of each frame and the gated
// output of one Transformer in one kernel (16-bit operands, dh = 64): O[token][h*64 + d].
struct BandLaunch {
  int dtype;
  const void* XH;           // [NB * BT][D] x^ (normalised unless rowss is given)
  const void* W;            // [3*H*64 + 64][D] W_qkv with the gate rows after q, k, v (the 16-bit repack)
  const float* gate_bias;   // [H]
  const float* cos;         // [64][32] rotary tables of the band positions
  const float* sin;
  const float* rowss;       // optional row statistics of x^ (row scale rs_mul / |x|)
  float rs_mul;
  float q_mul;              // log2 e: scores in log2 units
  void* O;                  // [NB * BT][H*64] gated attention output
  int32_t NB, BT, heads, D;
};
bool band_attn_supported(int dtype, int NB, int heads, int dh, int D);
hipError_t launch_band_attn(const BandLaunch& L, hipStream_t stream);

// y = gelu(x) elementwise with the device GELU of the feed-forward epilogues (test surface).
hipError_t launch_gelu(const float* x, float* y, int n, hipStream_t stream);

// Inverse-index average of the GLU output M [stems][B][ΣW][T] into the masks.
struct AverageLaunch {
  const float* M;
  float* out;
  const int32_t* inv_slot;   // [F*S][2]
  const float* inv_weight;   // [F*S]
  int32_t batch, stems, total, frames, n_freqs, channels, layout;
};
hipError_t launch_average(const AverageLaunch& L, hipStream_t stream);

// Out-projection, residual, feed-forward and both norms of one Transformer in one kernel
// (16-bit operands).  stream: the weights as fragment-ordered stages (block_stream_elems(D, I, FF)
// elements of the dtype, laid out by the creator).
struct BlockLaunch {
  int dtype;
  const void* O;            // [tokens][I] gated attention output
  const void* stream;
  const float* b1;          // [FF]
  const float* b2;          // [D]
  const float* gout;        // [D] gamma_out * sqrt(D)
  float* X;                 // [tokens][D] residual: x in, RMSNorm_out(x2) out
  void* XH;                 // [tokens][D] 16-bit copy for the next product
  int32_t tokens, D, I;
  int32_t xh_norm;          // 1: XH = x3 / |x3| * sqrt(D); 0: XH = x3
  int32_t ncu;              // compute units: a device pass is one 128-token block per compute unit
  float* part;              // block_part_bytes(D, tokens, ncu) bytes: partial sums of the tail
  // set by launch_block for each of its launches
  int64_t tok0;             // first token of the launch
  int32_t groups;           // hidden-chunk groups per 128 tokens (1: a block runs every chunk)
  int32_t main_blocks;      // blocks of whole device passes at the start of the grid
};
size_t block_part_bytes(int D, int64_t tokens, int ncu);
bool block_supported(int dtype, int D, int I, int FF);

// Geometry of the STFT / inverse STFT of a track cut into chunks (k_stft.hip).  A single signal is
// one chunk of its own length with no pad and no fades.
struct StftGeom {
  const float* wave;        // [S][L] track
  int32_t S, n_fft, hop, T; // channels, transform size, hop, frames per chunk (1 + chunk / hop)
  int32_t chunk0;           // first chunk of the current group
  int32_t no_fade;          // 1: every chunk weight 1 (a single signal)
  int64_t L, Lp, pad;       // track length, padded length, reflect pad on each side
  int64_t chunk, stride;    // chunk length and stride in samples
};
bool stft_supported(int n_fft);
hipError_t launch_stft(const StftGeom& G, int ngroup, float* spec, hipStream_t stream);
hipError_t launch_istft_frames(const StftGeom& G, int ngroup, const float* spec, const float* masks, int stems,
                               float* frames, hipStream_t stream);
hipError_t launch_ola(const StftGeom& G, const float* frames, int stems, int ngroup, int64_t lo, int64_t hi,
                      float* out, float* counter, hipStream_t stream);
hipError_t launch_finish(const StftGeom& G, int stems, const float* out, const float* counter, float* dst,
                         hipStream_t stream);
hipError_t launch_fill0(float* p, int64_t n, hipStream_t stream);
// Bytes of the static frame buffer of the allocation-free inverse STFT, and the current device's
// address of it (looked up once per device).
constexpr int64_t kIstftNoallocBytes = (int64_t)64 << 20;
hipError_t istft_noalloc_scratch(void** ptr);
int64_t block_stream_elems(int D, int I, int FF);
hipError_t launch_block(const BlockLaunch& L, hipStream_t stream);

}  // namespace mbr
