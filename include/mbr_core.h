/*
 * mbr_core.h — C ABI of the Mel-Band RoFormer mask-estimation core on AMD MI355X (gfx950).
 *
 * The core is the network between an STFT and its inverse in a music source separator:
 * complex stereo STFT bins in, per-bin complex masks out.  What it computes is stated on
 *   [P1] "Mel-Band RoFormer — architecture, inference hot path & RTX 3050 feasibility",
 *        sections "The forward chain", "The mel-band split, exactly", "The two transformers
 *        are not the same shape", "Parameter accounting";
 *   [P3] "Vocal Separation Core (Mel-Band RoFormer) — ONNX / fp16 / WebGPU", section
 *        "How to use" and its signature table (stft_repr -> masks, both [B, F*S, T, 2]);
 *   [P4] "Mel-Band RoFormer (vocals), ONNX for the GPU (float16 weights)", section "Graph"
 *        (the plane layout [B, S*2, F, T]);
 *   [P5] "@audio/neural-separate 0.4.0 -> 0.5.0", scripts/export-roformer.py (class Core)
 *        and roformer.js (the session shape {run, free}, null without a capable GPU).
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative MBR_E_* code; mbr_last_error() then describes the
 *     failure (per calling thread).  No C++ exception crosses this boundary.
 *   - Pointers named "host" are host memory, pointers named "dev" are device memory on the
 *     GPU that is current when the call is made.  The caller owns every pointer it passes.
 *   - A handle is bound to the device that was current at mbr_core_create; use it with
 *     that device current.  Calls on one handle must not overlap (the workspace is shared).
 */
#ifndef MBR_CORE_H
#define MBR_CORE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------------------ */
#define MBR_OK         0
#define MBR_E_ARG     (-1) /* null pointer, bad index, batch out of range                  */
#define MBR_E_CONFIG  (-2) /* invalid configuration: a band without bins, a bin in more than
                              two bands or in none, sizes out of range, unknown dtype/layout */
#define MBR_E_DEVICE  (-3) /* the current device is not a gfx950 (MI355X-class) GPU          */
#define MBR_E_HIP     (-4) /* a HIP runtime call failed                                      */
#define MBR_E_NOMEM   (-5) /* device or host allocation failed                              */

/* ---- enumerations ----------------------------------------------------------------- */
enum { MBR_F32 = 0, MBR_F16 = 1, MBR_BF16 = 2 };          /* weight / GEMM operand dtype    */
enum { MBR_IO_FS_T_C = 0, MBR_IO_SC_F_T = 1 };            /* boundary tensor layout         */
enum { MBR_KIND_MATRIX = 0, MBR_KIND_BIAS = 1, MBR_KIND_GAMMA = 2 };

/*
 * Configuration of one core.
 *   sample_rate, n_fft      STFT the bands are built for (F = n_fft/2 + 1 bins).
 *   audio_channels (S)      stereo = 2; merged into the frequency axis as pair = f*S + s.
 *   num_bands (NB)          Slaney-mel bands ([P1] "The mel-band split, exactly").
 *   dim (D), depth (L)      residual width and number of axial blocks (time + band each).
 *   heads (H), dim_head     attention heads; inner width H*dim_head ([P1] "Per Attention layer").
 *   ff_mult                 feed-forward hidden = ff_mult * D.
 *   mask_hidden_mult        mask-MLP hidden = mask_hidden_mult * D.
 *   mask_depth              number of Linear+Tanh layers before the last Linear of the mask MLP
 *                           (2 in every published configuration: three Linear layers).
 *   num_stems               mask heads sharing one trunk (1 = one set of masks).
 *   max_batch, frames (T)   largest batch a forward may use, frames per chunk.
 *   dtype                   MBR_F32: fp32 everywhere; MBR_F16 / MBR_BF16: weights and GEMM /
 *                           attention operands in that type, fp32 accumulation, softmax, norms
 *                           and residual stream.
 *   io_layout               MBR_IO_FS_T_C: [B, F*S, T, 2] (last axis re, im) ([P3]);
 *                           MBR_IO_SC_F_T: [B, S*2, F, T] (planes L re, L im, R re, R im) ([P4]).
 *   zero_dc                 1: the DC bin's masks are zero (the average gives that bin weight 0,
 *                           the zero_dc option of [P5]'s roformer export); 0: the plain average ([P1]).
 *   band_bins               NULL: Slaney-mel bands.  Else a host array of num_bands bin counts:
 *                           contiguous, non-overlapping bands that cover the F bins in order
 *                           (a band-split table of the kind [P2] "Evaluation record" describes
 *                           for its BS PolarFormer section: 62 bands over all 1025 bins).  Read
 *                           during the call only.
 */
typedef struct mbr_config {
  int32_t sample_rate;
  int32_t n_fft;
  int32_t audio_channels;
  int32_t num_bands;
  int32_t dim;
  int32_t depth;
  int32_t heads;
  int32_t dim_head;
  int32_t ff_mult;
  int32_t mask_hidden_mult;
  int32_t mask_depth;
  int32_t num_stems;
  int32_t max_batch;
  int32_t frames;
  int32_t dtype;
  int32_t io_layout;
  int32_t zero_dc;
  const int32_t* band_bins;
} mbr_config;

typedef struct mbr_core mbr_core;

/* Text of the last error on the calling thread ("" if none).  The string stays valid until
 * the next failing call on that thread. */
const char* mbr_last_error(void);

/* ---- weight inventory ------------------------------------------------------------- */
/*
 * The weights are a fixed list of tensors in canonical order, following the module tree of
 * [P1] "Parameter accounting" / "Per Attention layer" and [P5] class Core (Linear weights are
 * [out, in], row-major):
 *   for each band i (W_i = 2*S*bins_i):   norm.gamma [W_i], proj.weight [D, W_i], proj.bias [D]
 *   for each layer l, for axis in (time, band):
 *       attn.norm.gamma [D], attn.to_qkv.weight [3*H*dh, D], attn.to_gates.weight [H, D],
 *       attn.to_gates.bias [H], attn.to_out.weight [D, H*dh], ff.norm.gamma [D],
 *       ff.fc1.weight [FF, D], ff.fc1.bias [FF], ff.fc2.weight [D, FF], ff.fc2.bias [D],
 *       norm.gamma [D]
 *   for each stem, for each band i, for j in 0..mask_depth:
 *       mlp{j}.weight [out_j, in_j], mlp{j}.bias [out_j]
 *       with (in, out) = (D, MH), (MH, MH) ..., (MH, 2*W_i); the last layer's first W_i
 *       outputs are the GLU values and the second W_i its gates.
 * mbr_core_weight_count returns the number of tensors (or a negative error code).
 * mbr_core_weight_info writes tensor `index`'s shape: rank (1 or 2) to *ndim, sizes to dims[0..1]
 * (dims[1] = 1 for vectors) and its kind (MBR_KIND_*) to *kind.
 */
int mbr_core_weight_count(const mbr_config* cfg);
int mbr_core_weight_info(const mbr_config* cfg, int index, int* ndim, int64_t dims[2], int* kind);

/* ---- band tables ------------------------------------------------------------------ */
/*
 * Sizes of the tables of mbr_core_tables: *num_bands, *total_width (sum of W_i, features of
 * all bands), *n_freqs (F).
 */
int mbr_core_table_sizes(const mbr_config* cfg, int32_t* num_bands, int32_t* total_width, int32_t* n_freqs);
/*
 * The band tables of [P1] "The mel-band split, exactly": a binarised Slaney-mel filter bank with
 * DC forced into band 0 and Nyquist into the last band; each band's bins ascending, channels
 * interleaved (pair = bin*S + s); features = pair rank*2 + (re, im).  All buffers are host
 * memory the caller allocates (any may be NULL to skip it):
 *   band_bins     [NB]        bins in each band
 *   band_offset   [NB + 1]    first feature of each band in the concatenation of all bands
 *   gather_pair   [ΣW / 2]    pair index (bin*S + s) of every (band, pair rank) slot, bands in order
 *   inv_slot      [F*S*2]     for each pair p: the slots (into gather_pair) holding p, at most two;
 *                             entries 2p and 2p+1, -1 where a bin has only one band
 *   inv_weight    [F*S]       1 / (number of bands covering the pair's bin)
 *   bin_count     [F]         number of bands covering each bin (1 or 2)
 */
int mbr_core_tables(const mbr_config* cfg, int32_t* band_bins, int32_t* band_offset, int32_t* gather_pair,
                    int32_t* inv_slot, float* inv_weight, int32_t* bin_count);

/* ---- lifetime --------------------------------------------------------------------- */
/*
 * Build a core on the current device.  weights[i] is a DEVICE pointer to tensor i of the
 * inventory, stored in cfg->dtype (float32, float16 or bfloat16 bit patterns), row-major.
 * The library copies and repacks them (norm gains and the attention scale folded into the
 * following projections, per-band tiles padded, mask gates paired with their values), so the
 * caller may free them as soon as this returns.  Synchronous.  Allocates all device memory the
 * forward needs for up to cfg->max_batch chunks of cfg->frames frames.
 * Errors: MBR_E_ARG, MBR_E_CONFIG, MBR_E_DEVICE, MBR_E_HIP, MBR_E_NOMEM; *out is NULL then.
 */
int mbr_core_create(const mbr_config* cfg, const void* const* weights, int n_weights, mbr_core** out);

/*
 * One forward of the core ([P1] "The forward chain", from the mel gather to the division by
 * the band count).  stft_repr (dev, float32) and masks (dev, float32) are in cfg->io_layout:
 *   MBR_IO_FS_T_C: [batch, F*S, T, 2]       MBR_IO_SC_F_T: [batch, S*2, F, T]
 * with a leading stem axis after batch in masks when num_stems > 1.  1 <= batch <= max_batch.
 * Enqueued on `stream` (0 = the null stream); returns without waiting.  No allocation, no host
 * synchronisation and no atomics: the same input at the same batch size gives bitwise the same
 * masks.  Across batch sizes a chunk's masks agree to rounding, not bitwise: on the 16-bit path
 * with dim 384 or 512 the tokens after the last whole device pass sum their feed-forward in another fp32
 * order, and which tokens those are depends on the batch.  The core's workspace serves one forward
 * at a time: calls on one core must be ordered (one stream, or streams joined by events), never
 * concurrent.  The caller keeps both buffers alive until the stream has passed this work.  The
 * masks are not multiplied with the spectrum.
 */
int mbr_core_forward(mbr_core* core, const float* stft_repr_dev, float* masks_dev, int batch, hipStream_t stream);

/* Release the core's device memory.  NULL is accepted. */
void mbr_core_destroy(mbr_core* core);

/* ---- test taps -------------------------------------------------------------------- */
/*
 * Run the forward up to a stage and copy that stage's tensor (float32) to out_dev:
 *   stage 0            band embedding x, layout [NB][batch][T][D]
 *   stage 1 + k        x after Transformer k (k = 2*l for layer l's time axis, 2*l + 1 band axis)
 *   stage 1000         the GLU output of stem 0, layout [batch][ΣW][T] (feature-major)
 * mbr_core_debug_size gives the number of floats of a stage for a batch (negative on error).
 * Synchronous on `stream`.
 */
int64_t mbr_core_debug_size(const mbr_core* core, int batch, int stage);
int mbr_core_forward_debug(mbr_core* core, const float* stft_repr_dev, int batch, int stage, float* out_dev,
                           hipStream_t stream);

/* ---- per-kernel timing ------------------------------------------------------------ */
/* Kernel classes of one forward, in launch order. */
enum {
  MBR_K_GATHER = 0,      /* band gather + per-band normalisation                        */
  MBR_K_EMBED = 1,       /* per-band projection (grouped GEMM)                          */
  MBR_K_NORM = 2,        /* RMSNorm passes over the residual stream (+ attention gates)  */
  MBR_K_QKV = 3,         /* q/k/v projection with rotary                                 */
  MBR_K_ATTN_TIME = 4,   /* attention along frames                                       */
  MBR_K_ATTN_BAND = 5,   /* attention along bands                                        */
  MBR_K_OUT_PROJ = 6,    /* attention output projection + residual                       */
  MBR_K_FFN1 = 7,        /* feed-forward first layer + GELU                              */
  MBR_K_FFN2 = 8,        /* feed-forward second layer + residual                         */
  MBR_K_MASK_HIDDEN = 9, /* mask MLP hidden layers (grouped GEMM, tanh)                  */
  MBR_K_MASK_GLU = 10,   /* mask MLP last layer + GLU (grouped GEMM)                     */
  MBR_K_AVERAGE = 11,    /* inverse-index mask average                                   */
  MBR_K_BLOCK = 12,      /* 16-bit path: out-projection, residual, feed-forward and both
                            norms of a Transformer in one kernel (replaces 6, 7, 8)      */
  MBR_K_BAND_ATTN = 13,  /* 16-bit path: the band axis' q/k/v projection, rotary, attention
                            and gates in one kernel (replaces 3 and 5 on that axis)      */
  MBR_K_COUNT = 14
};
/*
 * The same forward as mbr_core_forward, with a HIP event pair recorded on `stream` around every
 * kernel launch; waits for the stream, then writes per class the summed device milliseconds
 * (ms_per_kind[MBR_K_COUNT]) and the number of launches (launches_per_kind[MBR_K_COUNT]), host
 * arrays.  Meant for measurement, not for the serving path (it creates events and synchronises).
 */
int mbr_core_forward_profiled(mbr_core* core, const float* stft_repr_dev, float* masks_dev, int batch,
                              hipStream_t stream, double* ms_per_kind, int32_t* launches_per_kind);

/* ---- kernel test surface ------------------------------------------------------------ */
/*
 * One dense GEMM through the library's matrix-core kernels, for tests and tile tuning:
 * C = A . B^T (+ bias), A [M, K] and B [N, K] row-major device arrays in `dtype` (MBR_F16 /
 * MBR_BF16 bit patterns or float32), bias [N] float32 device array or NULL, C [M, N] device array
 * (overwritten) in float32, or in `dtype` when out16 != 0 (16-bit dtypes only).  Needs N % 64 == 0
 * and K % 32 == 0 (K % 16 for MBR_F32).  `variant` picks a tile configuration of the 16-bit
 * kernel, 0 .. mbr_k_gemm_variants() - 1 (ignored for MBR_F32).  Asynchronous on `stream`.
 */
int mbr_k_gemm(int dtype, const void* a_dev, const void* b_dev, const float* bias_dev, void* c_dev, int M, int N,
               int K, int variant, int out16, hipStream_t stream);
int mbr_k_gemm_variants(void);
/*
 * y[i] = GELU(x[i]) = x * Phi(x) with the library's device error function (Abramowitz & Stegun
 * 7.1.26, |erf error| <= 1.5e-7), the one the feed-forward epilogues use.  x, y: n float32 device
 * values.  Asynchronous on `stream`.
 */
int mbr_k_gelu(const float* x_dev, float* y_dev, int n, hipStream_t stream);

/*
 * Gated scaled dot-product attention on 16-bit operands with the flash kernel of the core's time
 * axis (online softmax in fp32, the scores never stored), for q / k of width dqk and v of width dv:
 *   o[s][t][h*dv + d] = gate[s*n + t][h] * sum_j softmax_j(scale * q[s][h][t] . k[s][h][j]) v[s][h][j][d]
 * dv may be half of dqk: the attention of [P2] "Evaluation record", section "BS PolarFormer: the same
 * quality for a quarter of the arithmetic", part "Ported, and what it actually bought", whose polar
 * positional scheme doubles the depth of q and k and leaves v alone, and which asks for a fused
 * attention that accepts v narrower than q (the positional transform itself is the caller's: q and
 * k arrive transformed).
 *   q_dev, k_dev   [seqs][heads][npad][dqk] in dtype (MBR_F16 or MBR_BF16).
 *   vt_dev         [seqs][heads][dv][npad] in dtype: v transposed, positions contiguous.
 *   gates_dev      [seqs * n][heads] float32, or NULL for gates of 1.
 *   o_dev          [seqs][n][heads * dv] in dtype (written).
 * 1 <= n <= npad, npad a multiple of 128; (dqk, dv) = (32, 32), (64, 64) or (128, 64); scale > 0
 * (dqk^-1/2 for the usual scaling).  Rows n .. npad-1 of q and k and columns n .. npad-1 of vt are
 * read and must hold finite values (those keys get probability 0, but 0 x inf is not 0).  Returns
 * MBR_E_ARG on bad sizes, MBR_E_HIP if the launch fails.  Asynchronous on `stream`.
 */
int mbr_attention(int dtype, const void* q_dev, const void* k_dev, const void* vt_dev, const float* gates_dev,
                  void* o_dev, int seqs, int heads, int n, int npad, int dqk, int dv, float scale, hipStream_t stream);

/* Device bytes held by the core (weights + workspace). */
int64_t mbr_core_device_bytes(const mbr_core* core);

/* ---- around the core: STFT, masked inverse STFT, chunked separation ----------------- */
/*
 * STFT of a waveform as [P1] "The forward chain" takes it: centred (the signal reflected about its
 * end samples by n_fft/2 on both sides), periodic Hann window of n_fft, hop `hop`, one-sided.
 *   wave_dev       [channels][length] float32 device array (read).
 *   stft_repr_dev  [1][F*channels][T][2] float32 device array (written), F = n_fft/2 + 1,
 *                  T = 1 + length / hop, pair = f*channels + s, last axis (re, im): the core's
 *                  MBR_IO_FS_T_C input.
 * n_fft a power of two in 16..4096, 1 <= hop <= n_fft / 2, length >= 2.  Asynchronous on stream.
 * Returns MBR_E_ARG on bad sizes, MBR_E_HIP if a launch fails.
 */
int mbr_stft(const float* wave_dev, int channels, int64_t length, int n_fft, int hop, float* stft_repr_dev,
             hipStream_t stream);
/*
 * Inverse of mbr_stft after the complex product with masks ([P1] "The forward chain": multiply
 * the original complex STFT, inverse STFT): out[stem][s] = iSTFT(stft_repr x masks[stem]) of
 * `length` samples, the windowed overlap-add divided by the summed squared window.
 *   stft_repr_dev  [1][F*channels][T][2] (mbr_stft's layout), T = 1 + length / hop.
 *   masks_dev      [stems][F*channels][T][2] (the core's output for one chunk).
 *   workspace_dev  mbr_istft_workspace_size(channels, n_fft, T, stems) bytes of device memory,
 *                  owned by the caller; contents need not be initialised and are overwritten.
 *   out_dev        [stems][channels][length] float32 (written).
 */
int64_t mbr_istft_workspace_size(int channels, int n_fft, int frames, int stems);
int mbr_istft_masked(const float* stft_repr_dev, const float* masks_dev, int stems, int channels, int64_t length,
                     int n_fft, int hop, void* workspace_dev, float* out_dev, hipStream_t stream);
/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): mbr_istft_masked with no workspace argument.  The
 * frame buffer is a static device array of MBR_ISTFT_NOALLOC_MAX_BYTES bytes in the library, one
 * copy per GPU, held until the process ends; its address is looked up on the first call on each
 * device.  Arguments, layouts and results as mbr_istft_masked (the same kernels; the outputs are
 * bitwise equal).  Calls allocate nothing and clear nothing they do not write first.  Every call
 * on one GPU shares that GPU's buffer, so calls that overlap on one GPU (different streams or
 * threads without ordering between them) race and give wrong results: order them.
 * Returns MBR_E_ARG when stems * channels * (1 + length / hop) * n_fft * 4 exceeds
 * MBR_ISTFT_NOALLOC_MAX_BYTES (64 MiB: about 41 s of stereo audio at n_fft 2048, hop 441, one
 * stem) or on bad sizes, MBR_E_HIP if the buffer lookup or a launch fails.
 */
#define MBR_ISTFT_NOALLOC_MAX_BYTES ((int64_t)64 << 20)
int mbr_istft_masked_noalloc(const float* stft_repr_dev, const float* masks_dev, int stems, int channels,
                             int64_t length, int n_fft, int hop, float* out_dev, hipStream_t stream);
/*
 * Separation of one track by chunks ([P1] "Verified inference hot path", steps 3-9): chunk =
 * (core frames - 1) * hop samples, stride int(0.9 * chunk), border = chunk - stride; a track
 * longer than two borders is reflect-padded by one border on each side; each chunk (its tail
 * reflected when it holds more than half a chunk, else zero-padded) goes STFT -> core -> masks x
 * STFT -> inverse STFT; the estimates are weighted by linear fades of chunk / 10 (none before the
 * first chunk, none after the last), summed, divided by the summed fades (at least 1e-8), and the
 * padding is cropped.  Chunks go through the core max_batch at a time.
 *   core           created with io_layout MBR_IO_FS_T_C and audio_channels = the track's channels;
 *                  its n_fft is the STFT's.
 *   wave_dev       [channels][length] float32.
 *   workspace_dev  mbr_separate_workspace_size(core, length, hop) bytes, caller-owned, any content.
 *   out_dev        [stems][channels][length] float32 (written).
 * The core's frames must give a chunk of at least 20 samples, 1 <= hop <= n_fft / 2.  Returns
 * MBR_E_ARG on bad sizes or a core of another io_layout, MBR_E_HIP if a launch fails; the work
 * is asynchronous on `stream` and the workspace must stay allocated until it completes.
 */
int64_t mbr_separate_workspace_size(const mbr_core* core, int64_t length, int hop);
int mbr_separate(mbr_core* core, const float* wave_dev, int64_t length, int hop, void* workspace_dev,
                 float* out_dev, hipStream_t stream);
/*
 * mbr_separate with the chunk stride chosen by the caller, in samples: 0 gives int(0.9 * chunk)
 * (mbr_separate itself); chunk / 2 gives the segmenting of [P4] "Graph" (8 s segments every 4 s,
 * faded over 0.8 s, the input reflected out at the ends, as the training repository's demix runs
 * with two overlaps).  Everything else as mbr_separate: the border (reflect pad) is chunk - stride,
 * the fades chunk / 10, the summed fades divide the sum.  1 <= stride <= chunk - chunk / 10 (so every
 * sample of the padded track has a chunk of weight 1 over it), else MBR_E_ARG.  The workspace size
 * depends on the stride.
 */
int64_t mbr_separate_workspace_size_strided(const mbr_core* core, int64_t length, int hop, int64_t stride);
int mbr_separate_strided(mbr_core* core, const float* wave_dev, int64_t length, int hop, int64_t stride,
                         void* workspace_dev, float* out_dev, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MBR_CORE_H */
