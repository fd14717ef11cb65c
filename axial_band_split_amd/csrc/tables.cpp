// Host tables of the Mel-Band RoFormer core.
//
// Band membership follows [P1] "Mel-Band RoFormer — architecture, inference hot path & RTX 3050
// feasibility", section "The mel-band split, exactly": a Slaney-mel triangular filter bank over
// the STFT bins (fmin 0, fmax sr/2, n_mels + 2 points equally spaced on the mel scale), a bin is
// in a band when that band's triangle is positive at the bin, DC is forced into the first band
// and Nyquist into the last.  The triangle of band i is positive exactly on the open interval
// between mel points i and i+2, so membership is decided by that interval test (no weights are
// formed).  Channels interleave inside a band (pair = bin*S + s) and each pair contributes its
// real and imaginary part as two features ([P1] "The forward chain": fold the complex axis into
// channels).  The per-bin band count divides the scattered masks ([P1] same section).
#include "tables.h"

#include <cmath>
#include <cstdio>

namespace mbr {

namespace {

// Slaney's mel scale: 3 mels per 200 Hz below 1 kHz, then 27 mels per factor 6.4.
double hz_to_mel(double f) {
  if (f < 1000.0) return f * 3.0 / 200.0;
  return 15.0 + std::log(f / 1000.0) * 27.0 / std::log(6.4);
}
double mel_to_hz(double m) {
  if (m < 15.0) return m * 200.0 / 3.0;
  return 1000.0 * std::exp((m - 15.0) * std::log(6.4) / 27.0);
}

}  // namespace

int validate_config(const mbr_config& c, std::string* err) {
  auto bad = [&](const char* what) {
    *err = std::string("invalid config: ") + what;
    return MBR_E_CONFIG;
  };
  if (c.sample_rate <= 0) return bad("sample_rate must be > 0");
  if (c.n_fft < 4 || c.n_fft % 2) return bad("n_fft must be even and >= 4");
  if (c.audio_channels < 1 || c.audio_channels > 8) return bad("audio_channels must be in 1..8");
  if (c.num_bands < 1 || c.num_bands > 512) return bad("num_bands must be in 1..512");
  if (c.dim < 64 || c.dim > 1024 || c.dim % 64) return bad("dim must be a multiple of 64 in 64..1024");
  if (c.depth < 1 || c.depth > 64) return bad("depth must be in 1..64");
  if (c.dim_head != 32 && c.dim_head != 64) return bad("dim_head must be 32 or 64");
  if (c.heads < 1 || c.heads > 32) return bad("heads must be in 1..32");
  if ((c.heads * c.dim_head) % 64) return bad("heads*dim_head must be a multiple of 64");
  if (c.ff_mult < 1 || c.ff_mult > 8) return bad("ff_mult must be in 1..8");
  if (c.mask_hidden_mult < 1 || c.mask_hidden_mult > 8) return bad("mask_hidden_mult must be in 1..8");
  if (c.mask_depth < 1 || c.mask_depth > 8) return bad("mask_depth must be in 1..8");
  if (c.num_stems < 1 || c.num_stems > 8) return bad("num_stems must be in 1..8");
  if (c.max_batch < 1 || c.max_batch > 64) return bad("max_batch must be in 1..64");
  if (c.frames < 1 || c.frames > 8192) return bad("frames must be in 1..8192");
  if (c.dtype != MBR_F32 && c.dtype != MBR_F16 && c.dtype != MBR_BF16) return bad("unknown dtype");
  if (c.io_layout != MBR_IO_FS_T_C && c.io_layout != MBR_IO_SC_F_T) return bad("unknown io_layout");
  if (c.zero_dc != 0 && c.zero_dc != 1) return bad("zero_dc must be 0 or 1");
  if (c.band_bins) {
    int64_t sum = 0;
    for (int i = 0; i < c.num_bands; ++i) {
      if (c.band_bins[i] < 1) return bad("every band of band_bins needs at least one bin");
      sum += c.band_bins[i];
    }
    if (sum != c.n_fft / 2 + 1) return bad("band_bins must add up to n_fft/2 + 1");
  }
  return MBR_OK;
}

int build_bands(const mbr_config& cfg, Bands* out, std::string* err) {
  int rc = validate_config(cfg, err);
  if (rc) return rc;
  const int F = cfg.n_fft / 2 + 1, NB = cfg.num_bands, S = cfg.audio_channels;
  const double top = hz_to_mel(cfg.sample_rate / 2.0);
  std::vector<double> pts(NB + 2);
  for (int j = 0; j < NB + 2; ++j) pts[j] = mel_to_hz(top * j / (NB + 1));
  Bands b;
  b.n_freqs = F;
  b.channels = S;
  b.bins.assign(NB, {});
  b.count.assign(F, 0);
  for (int i = 0, k0 = 0; cfg.band_bins && i < NB; k0 += cfg.band_bins[i++])   // explicit table
    for (int k = k0; k < k0 + cfg.band_bins[i]; ++k) b.bins[i].push_back(k);
  for (int i = 0; i < NB; ++i) {
    for (int k = 0; k < F && !cfg.band_bins; ++k) {
      double hz = (double)k * cfg.sample_rate / cfg.n_fft;
      bool in = pts[i] < hz && hz < pts[i + 2];
      if (i == 0 && k == 0) in = true;
      if (i == NB - 1 && k == F - 1) in = true;
      if (in) b.bins[i].push_back(k);
    }
    if (b.bins[i].empty()) {
      *err = "invalid config: band " + std::to_string(i) + " covers no frequency bin";
      return MBR_E_CONFIG;
    }
    for (int k : b.bins[i]) b.count[k]++;
  }
  for (int k = 0; k < F; ++k) {
    if (b.count[k] == 0) {
      *err = "invalid config: bin " + std::to_string(k) + " is in no band";
      return MBR_E_CONFIG;
    }
    if (b.count[k] > 2) {
      *err = "invalid config: bin " + std::to_string(k) + " is in more than two bands";
      return MBR_E_CONFIG;
    }
  }
  b.width.resize(NB);
  b.offset.assign(NB + 1, 0);
  for (int i = 0; i < NB; ++i) {
    b.width[i] = 2 * S * (int)b.bins[i].size();
    b.offset[i + 1] = b.offset[i] + b.width[i];
    for (int k : b.bins[i])
      for (int s = 0; s < S; ++s) b.gather_pair.push_back(k * S + s);
  }
  b.inv_slot.assign((size_t)F * S * 2, -1);
  for (int slot = 0; slot < (int)b.gather_pair.size(); ++slot) {
    int p = b.gather_pair[slot];
    if (b.inv_slot[2 * p] < 0)
      b.inv_slot[2 * p] = slot;
    else
      b.inv_slot[2 * p + 1] = slot;
  }
  b.inv_weight.resize((size_t)F * S);
  for (int p = 0; p < F * S; ++p) b.inv_weight[p] = (cfg.zero_dc && p / S == 0) ? 0.0f : 1.0f / (float)b.count[p / S];
  *out = std::move(b);
  return MBR_OK;
}

std::vector<WeightInfo> inventory(const mbr_config& c, const Bands& bands) {
  std::vector<WeightInfo> v;
  const int64_t D = c.dim, I = (int64_t)c.heads * c.dim_head, H = c.heads, FF = (int64_t)c.ff_mult * c.dim,
                MH = (int64_t)c.mask_hidden_mult * c.dim;
  auto vec = [&](std::string n, int64_t len, int kind) { v.push_back({std::move(n), 1, len, 1, kind}); };
  auto mat = [&](std::string n, int64_t r, int64_t cols) { v.push_back({std::move(n), 2, r, cols, MBR_KIND_MATRIX}); };
  for (int i = 0; i < bands.num_bands(); ++i) {
    std::string p = "band" + std::to_string(i) + ".";
    vec(p + "norm.gamma", bands.width[i], MBR_KIND_GAMMA);
    mat(p + "proj.weight", D, bands.width[i]);
    vec(p + "proj.bias", D, MBR_KIND_BIAS);
  }
  for (int l = 0; l < c.depth; ++l) {
    for (int ax = 0; ax < 2; ++ax) {
      std::string p = "layer" + std::to_string(l) + (ax == 0 ? ".time." : ".band.");
      vec(p + "attn.norm.gamma", D, MBR_KIND_GAMMA);
      mat(p + "attn.to_qkv.weight", 3 * I, D);
      mat(p + "attn.to_gates.weight", H, D);
      vec(p + "attn.to_gates.bias", H, MBR_KIND_BIAS);
      mat(p + "attn.to_out.weight", D, I);
      vec(p + "ff.norm.gamma", D, MBR_KIND_GAMMA);
      mat(p + "ff.fc1.weight", FF, D);
      vec(p + "ff.fc1.bias", FF, MBR_KIND_BIAS);
      mat(p + "ff.fc2.weight", D, FF);
      vec(p + "ff.fc2.bias", D, MBR_KIND_BIAS);
      vec(p + "norm.gamma", D, MBR_KIND_GAMMA);
    }
  }
  for (int s = 0; s < c.num_stems; ++s) {
    for (int i = 0; i < bands.num_bands(); ++i) {
      std::vector<int64_t> dims;
      dims.push_back(D);
      for (int j = 0; j < c.mask_depth; ++j) dims.push_back(MH);
      dims.push_back(2 * (int64_t)bands.width[i]);
      for (size_t j = 0; j + 1 < dims.size(); ++j) {
        std::string p = "stem" + std::to_string(s) + ".band" + std::to_string(i) + ".mlp" + std::to_string(j) + ".";
        mat(p + "weight", dims[j + 1], dims[j]);
        vec(p + "bias", dims[j + 1], MBR_KIND_BIAS);
      }
    }
  }
  return v;
}

// Rotary embedding of the head dimension: pair (2j, 2j+1) of a query or key at position pos is
// rotated by pos * 10000^(-2j/dh).  The pages name the rotary module but print neither its base nor
// its frequencies; 10000 with these inverse frequencies is the rotary embedding's usual form.
void rope_tables(int n, int dh, std::vector<float>* cos_t, std::vector<float>* sin_t) {
  const int half = dh / 2;
  cos_t->resize((size_t)n * half);
  sin_t->resize((size_t)n * half);
  for (int pos = 0; pos < n; ++pos)
    for (int j = 0; j < half; ++j) {
      double ang = (double)pos * std::pow(10000.0, -2.0 * j / dh);
      (*cos_t)[(size_t)pos * half + j] = (float)std::cos(ang);
      (*sin_t)[(size_t)pos * half + j] = (float)std::sin(ang);
    }
}

}  // namespace mbr
