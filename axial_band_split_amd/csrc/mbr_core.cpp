// C ABI of the Mel-Band RoFormer core: configuration, weight repacking, workspace and the launch
// sequence of one forward.  The functions declared in include/mbr_core.h live here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mbr_core.h"
#include "kernels.h"
#include "tables.h"

using namespace mbr;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                                         \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(MBR_E_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

int round_up(int x, int m) { return (x + m - 1) / m * m; }

size_t dtype_size(int dt) { return dt == MBR_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------------- host numerics
float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
uint16_t float_to_bf16(float f) {  // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

std::vector<double> to_double(const std::vector<char>& raw, int dt, size_t n) {
  std::vector<double> out(n);
  if (dt == MBR_F32) {
    const float* p = (const float*)raw.data();
    for (size_t i = 0; i < n; ++i) out[i] = p[i];
  } else if (dt == MBR_F16) {
    const _Float16* p = (const _Float16*)raw.data();
    for (size_t i = 0; i < n; ++i) out[i] = (double)(float)p[i];
  } else {
    const uint16_t* p = (const uint16_t*)raw.data();
    for (size_t i = 0; i < n; ++i) out[i] = bf16_to_float(p[i]);
  }
  return out;
}

// Append values (double) in dtype to a byte buffer, 256-byte aligned start; returns element offset.
struct Packer {
  int dt;
  std::vector<char> bytes;
  size_t append(const std::vector<double>& v) {
    size_t esz = dtype_size(dt);
    size_t pos = bytes.size();
    size_t aligned = (pos + 255) / 256 * 256;
    bytes.resize(aligned + v.size() * esz);
    char* p = bytes.data() + aligned;
    for (size_t i = 0; i < v.size(); ++i) {
      float f = (float)v[i];
      if (dt == MBR_F32) {
        std::memcpy(p + 4 * i, &f, 4);
      } else if (dt == MBR_F16) {
        _Float16 h = (_Float16)f;
        std::memcpy(p + 2 * i, &h, 2);
      } else {
        uint16_t b = float_to_bf16(f);
        std::memcpy(p + 2 * i, &b, 2);
      }
    }
    return aligned / esz;
  }
};
struct FPacker {  // fp32 side tables (biases, gains, gate weights)
  std::vector<float> v;
  size_t append(const std::vector<double>& x) {
    size_t pos = (v.size() + 63) / 64 * 64;
    v.resize(pos + x.size());
    for (size_t i = 0; i < x.size(); ++i) v[pos + i] = (float)x[i];
    return pos;
  }
};

struct TransformerW {
  size_t wqkv, wout, w1, w2;          // element offsets in the dtype weight block
  size_t bstream = 0;                 // fused post-attention kernel: fragment-ordered weight stages
  size_t wg, bg, b1, b2, gout;        // float offsets
};
struct MaskW {
  std::vector<size_t> w;              // per layer: offset of band 0's matrix (bands contiguous per layer)
  std::vector<std::vector<size_t>> wband;  // [layer][band] element offsets
  std::vector<std::vector<size_t>> bband;  // [layer][band] float offsets
};

}  // namespace

struct mbr_core {
  mbr_config cfg;
  Bands bands;
  int device = 0;
  int ncu = 256;                      // compute units of the device
  int NB = 0, D = 0, H = 0, DH = 0, I = 0, FF = 0, MH = 0, T = 0, Tp = 0, Bmax = 0, total = 0;
  std::vector<int> kpad, kcol, wp;    // per band: padded K of the embedding, U column block, mask N/2
  // 16-bit GEMM tile configuration per launch kind (k_gemm2.hip variants)
  int v_embed = 0, v_qkv = 0, v_out = 0, v_ffn1 = 0, v_ffn2 = 0, v_mask = 0, v_glu = 0;
  int glu_blk = 16;                   // value / gate pairing block of the last mask layer
  bool use_block = false;             // 16-bit path with the fused post-attention kernel
  bool use_band = false;              // 16-bit path: band axis' projection and attention in one kernel
  bool use_embed = false;             // 16-bit path: band gather and embedding in one kernel
  int kpad_total = 0, kpad_max = 0;
  // device memory
  char* wdev = nullptr;               // dtype weights
  float* fdev = nullptr;              // fp32 side tables
  size_t emb_w = 0, emb_b = 0;
  std::vector<size_t> emb_wband;
  size_t emb_frag = 0;                // fused embedding: fragment-ordered band weights, all bands
  std::vector<int32_t> emb_foff;      // per band: element offset of its fragments from emb_frag
  std::vector<TransformerW> tw;
  std::vector<MaskW> mw;              // per stem
  void* ws = nullptr;                 // workspace block
  size_t ws_bytes = 0, w_bytes = 0, f_bytes = 0;
  float* X = nullptr;
  void* XH = nullptr;
  float* part = nullptr;              // fused post-attention kernel: partial sums of the last tokens
  float* gates = nullptr;
  void* U = nullptr;
  void *qt = nullptr, *kt = nullptr, *vt = nullptr, *qb = nullptr, *kb = nullptr, *vb = nullptr;
  void* O = nullptr;
  void* H1 = nullptr;
  void* H2 = nullptr;
  float* Mglu = nullptr;
  // row partial sums of squares (16-bit path), [tokens][D/64]
  float* ssA = nullptr;   // of the residual stream x after a feed-forward (before the output norm)
  float* ssB = nullptr;   // of x * gamma_out: the next attention's normalised input
  float* ssC = nullptr;   // of x after the attention residual: the feed-forward's normalised input
  // tables
  int32_t* band_info = nullptr;
  int32_t* gather_pair = nullptr;
  int32_t* emb_woff = nullptr;        // [NB] (fused embedding)
  int32_t* band_order = nullptr;      // [NB] bands, widest first (fused embedding)
  int32_t* inv_slot = nullptr;
  float* inv_weight = nullptr;
  float *cos_t = nullptr, *sin_t = nullptr, *cos_b = nullptr, *sin_b = nullptr;
  // grouped GEMM descriptors
  GemmGroup* groups = nullptr;
  GemmTile* tiles = nullptr;
  int g_embed = 0, t_embed = 0, n_embed = 0;
  // mask head per layer: tile start and count of its one grouped launch over stems x bands
  std::vector<int> t_mask, n_mask;
  char* tables_dev = nullptr;
};

namespace {

int check_device(int* dev, int* ncu) {
  HIP_TRY(hipGetDevice(dev));
  hipDeviceProp_t p;
  HIP_TRY(hipGetDeviceProperties(&p, *dev));
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return fail(MBR_E_DEVICE, std::string("device is ") + p.gcnArchName + ", this library is built for gfx950");
  *ncu = p.multiProcessorCount;
  return MBR_OK;
}

int setup_tables_and_groups(mbr_core* c) {
  const mbr_config& cfg = c->cfg;
  const Bands& bd = c->bands;
  // band info [NB][4]
  std::vector<int32_t> info(c->NB * 4);
  for (int i = 0; i < c->NB; ++i) {
    info[4 * i + 0] = bd.offset[i];
    info[4 * i + 1] = bd.width[i];
    info[4 * i + 2] = c->kpad[i];
    info[4 * i + 3] = c->kcol[i];
  }
  std::vector<float> ct, st, cb, sb;
  rope_tables(c->Tp, c->DH, &ct, &st);
  rope_tables(64, c->DH, &cb, &sb);

  // grouped GEMM descriptors
  std::vector<GemmGroup> groups;
  std::vector<GemmTile> tiles;
  const bool f32 = cfg.dtype == MBR_F32;
  auto add_tiles = [&](int group, int N, int variant) {
    const int TM = f32 ? 128 : gemm2_tile_rows(variant), TN = f32 ? 128 : gemm2_tile_cols(variant);
    const int MT = (c->Bmax * c->T + TM - 1) / TM;  // row tiles for the largest batch
    for (int m = 0; m < MT; ++m)
      for (int n = 0; n < (N + TN - 1) / TN; ++n) tiles.push_back({group, m * TM, n * TN, 0});
  };
  c->g_embed = 0;
  c->t_embed = 0;
  for (int i = 0; i < (c->use_embed ? 0 : c->NB); ++i) {
    GemmGroup g{};
    g.a_off0 = 0;
    g.a_offb = c->kcol[i];
    g.b_off = (int64_t)c->emb_wband[i];
    g.c_off0 = 0;
    g.c_offb = (int64_t)i * c->D;
    g.bias_off = (int64_t)c->emb_b + (int64_t)i * c->D;
    g.N = c->D;
    g.K = c->kpad[i];
    g.lda = c->kpad[i];
    g.ldb = c->kpad[i];
    g.e0 = i;          // global rows of this band start at i * (batch * frames)
    groups.push_back(g);
    add_tiles((int)groups.size() - 1, g.N, c->v_embed);
  }
  c->n_embed = (int)tiles.size();
  {
    // the embedding's K differs per band (32 .. 544 at the vocals shape): longest K first, dealt so
    // that each XCD's contiguous run of the table (the kernel gives each XCD one run, in order)
    // holds every 8th tile of that order
    std::vector<GemmTile> t(tiles.begin() + c->t_embed, tiles.begin() + c->n_embed);
    std::stable_sort(t.begin(), t.end(),
                     [&](const GemmTile& a, const GemmTile& b) { return groups[a.group].K > groups[b.group].K; });
    const int nb = (int)t.size(), per = nb >> 3, rem = nb & 7;
    for (int i = 0; i < nb; ++i) {
      const int x = i & 7, slot = i >> 3;
      tiles[c->t_embed + x * per + std::min(x, rem) + slot] = t[i];
    }
  }
  // mask head: one grouped launch per layer covering every stem and band (a band's stems adjacent,
  // so at the first layer they share the A panel of that band's rows).  Hidden layers of stem s
  // live at band block s * NB + i of H1 / H2; the first layer reads x (shared by the stems).
  const int nl = cfg.mask_depth + 1;
  c->t_mask.assign(nl, 0);
  c->n_mask.assign(nl, 0);
  for (int j = 0; j < nl; ++j) {
    c->t_mask[j] = (int)tiles.size();
    for (int i = 0; i < c->NB; ++i) {
      for (int s = 0; s < cfg.num_stems; ++s) {
        GemmGroup g{};
        const int K = j == 0 ? c->D : c->MH;
        g.a_off0 = 0;
        g.a_offb = (int64_t)(j == 0 ? i : s * c->NB + i) * K;
        g.b_off = (int64_t)c->mw[s].wband[j][i];
        g.bias_off = (int64_t)c->mw[s].bband[j][i];
        g.K = K;
        g.lda = K;
        g.ldb = K;
        if (j < nl - 1) {
          g.N = c->MH;
          g.c_off0 = 0;
          g.c_offb = (int64_t)(s * c->NB + i) * c->MH;
          g.e0 = i;          // row statistics of x (the first layer's row scale) are per band
        } else {
          g.N = 2 * c->wp[i];
          g.c_off0 = 0;
          g.c_offb = (int64_t)s * c->total;   // stem block of the GLU output, times rows (B*T)
          g.e0 = bd.offset[i];
          g.e1 = bd.width[i];
        }
        groups.push_back(g);
        add_tiles((int)groups.size() - 1, g.N, j < nl - 1 ? c->v_mask : c->v_glu);
      }
    }
    c->n_mask[j] = (int)tiles.size() - c->t_mask[j];
  }

  // one device block for all tables
  size_t off = 0;
  auto place = [&](size_t bytes) {
    size_t o = (off + 255) / 256 * 256;
    off = o + bytes;
    return o;
  };
  // fused embedding: band weight offsets and the bands widest first
  std::vector<int32_t> order(c->NB);
  for (int i = 0; i < c->NB; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return c->kpad[a] > c->kpad[b]; });
  std::vector<int32_t> woff = c->emb_foff;
  woff.resize(c->NB, 0);
  size_t o_woff = place(woff.size() * 4), o_ord = place(order.size() * 4);
  size_t o_info = place(info.size() * 4), o_gp = place(bd.gather_pair.size() * 4),
         o_inv = place(bd.inv_slot.size() * 4), o_w = place(bd.inv_weight.size() * 4), o_ct = place(ct.size() * 4),
         o_st = place(st.size() * 4), o_cb = place(cb.size() * 4), o_sb = place(sb.size() * 4),
         o_g = place(groups.size() * sizeof(GemmGroup)), o_t = place(tiles.size() * sizeof(GemmTile));
  std::vector<char> host(off);
  std::memcpy(host.data() + o_woff, woff.data(), woff.size() * 4);
  std::memcpy(host.data() + o_ord, order.data(), order.size() * 4);
  std::memcpy(host.data() + o_info, info.data(), info.size() * 4);
  std::memcpy(host.data() + o_gp, bd.gather_pair.data(), bd.gather_pair.size() * 4);
  std::memcpy(host.data() + o_inv, bd.inv_slot.data(), bd.inv_slot.size() * 4);
  std::memcpy(host.data() + o_w, bd.inv_weight.data(), bd.inv_weight.size() * 4);
  std::memcpy(host.data() + o_ct, ct.data(), ct.size() * 4);
  std::memcpy(host.data() + o_st, st.data(), st.size() * 4);
  std::memcpy(host.data() + o_cb, cb.data(), cb.size() * 4);
  std::memcpy(host.data() + o_sb, sb.data(), sb.size() * 4);
  std::memcpy(host.data() + o_g, groups.data(), groups.size() * sizeof(GemmGroup));
  std::memcpy(host.data() + o_t, tiles.data(), tiles.size() * sizeof(GemmTile));
  HIP_TRY(hipMalloc(&c->tables_dev, off));
  HIP_TRY(hipMemcpy(c->tables_dev, host.data(), off, hipMemcpyHostToDevice));
  char* b = c->tables_dev;
  c->emb_woff = (int32_t*)(b + o_woff);
  c->band_order = (int32_t*)(b + o_ord);
  c->band_info = (int32_t*)(b + o_info);
  c->gather_pair = (int32_t*)(b + o_gp);
  c->inv_slot = (int32_t*)(b + o_inv);
  c->inv_weight = (float*)(b + o_w);
  c->cos_t = (float*)(b + o_ct);
  c->sin_t = (float*)(b + o_st);
  c->cos_b = (float*)(b + o_cb);
  c->sin_b = (float*)(b + o_sb);
  c->groups = (GemmGroup*)(b + o_g);
  c->tiles = (GemmTile*)(b + o_t);
  return MBR_OK;
}

// Weights of the fused post-attention kernel (k_block.hip) as the stages it copies into LDS, each
// stage D/8 fragments of 64 lanes x 8 elements in the order the lanes read them.  A fragment is
// the A operand of one 16 x 16 x 32 product: lane l supplies row l % 16 and K elements
// 8(l/16) .. 8(l/16)+7.
//   stages 0 .. I/64-1: out-projection, K step ks of 2, tile t of D/16 (rows 16t..): W_out[row][k]
//   stage I/64 + c:     W_1 rows of hidden chunk c (fragment 2s + u: rows 32c + 16u.., K step s of
//                       D/32) with the columns permuted to the accumulators' row order, then W_2
//                       columns of chunk c-2 (fragment D/16 + t: rows 16t..) permuted to the order the
//                       hidden tiles hold their rows, times 1/2 (the kernel's hidden layer holds
//                       twice the GELU).
// The accumulator of a 16 x 16 product holds in lane l rows 4(l/16) + v (v = 0..3); read as a B
// operand, K step s of the residual takes tiles 2s and 2s+1, i.e. for lane group q = l/16 and
// element e the row perm(s, q, e) = 32s + 16(e/4) + 4q + e%4, and the hidden chunk (two tiles) the
// row 16(e/4) + 4q + e%4.
std::vector<double> block_stream(int D, int I, int FF, const std::vector<double>& wout,
                                 const std::vector<double>& w1g, const std::vector<double>& w2) {
  const int DT = D / 16, KO = I / 64, NCH = FF / 32;
  const size_t stage = (size_t)D * 64;
  std::vector<double> out((size_t)(KO + NCH + 2) * stage, 0.0);
  auto perm = [](int s, int q, int e) { return 32 * s + 16 * (e / 4) + 4 * q + e % 4; };
  for (int st = 0; st < KO; ++st)
    for (int ks = 0; ks < 2; ++ks)
      for (int t = 0; t < DT; ++t)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) {
            const int row = 16 * t + l % 16, k = 64 * st + 32 * ks + 8 * (l / 16) + e;
            out[st * stage + ((size_t)(ks * DT + t) * 64 + l) * 8 + e] = wout[(size_t)row * I + k];
          }
  for (int c = 0; c <= NCH + 1; ++c) {
    const size_t base = (size_t)(KO + c) * stage;
    if (c < NCH)
      for (int s = 0; s < D / 32; ++s)
        for (int u = 0; u < 2; ++u)
          for (int l = 0; l < 64; ++l)
            for (int e = 0; e < 8; ++e)
              out[base + ((size_t)(2 * s + u) * 64 + l) * 8 + e] =
                  w1g[(size_t)(32 * c + 16 * u + l % 16) * D + perm(s, l / 16, e)];
    if (c > 1)
      for (int t = 0; t < DT; ++t)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e)
            out[base + ((size_t)(DT + t) * 64 + l) * 8 + e] =
                0.5 * w2[(size_t)(16 * t + l % 16) * FF + 32 * (c - 2) + perm(0, l / 16, e)];
  }
  return out;
}

// One band's embedding weights (m: D rows x kp columns) in the order the fused embedding kernel
// (k_embed.hip) reads them: wave w of 4 (features D/4 w ..), K step ks of 16, tile ft of 32
// features, then 64 lanes x 8 elements of the A operand of a 32 x 32 x 16 product (lane l: feature
// D/4 w + 32 ft + l % 32, K elements 16 ks + 8(l/32) ..).
std::vector<double> embed_stream(int D, int kp, const std::vector<double>& m) {
  std::vector<double> out((size_t)D * kp);
  const int fpw = D / 4, ft_n = fpw / 32;
  size_t o = 0;
  for (int w = 0; w < 4; ++w)
    for (int ks = 0; ks < kp / 16; ++ks)
      for (int ft = 0; ft < ft_n; ++ft)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) out[o++] = m[(size_t)(fpw * w + 32 * ft + l % 32) * kp + 16 * ks + 8 * (l / 32) + e];
  return out;
}

int repack_weights(mbr_core* c, const std::vector<std::vector<double>>& W) {
  const mbr_config& cfg = c->cfg;
  const Bands& bd = c->bands;
  const int D = c->D, I = c->I, H = c->H, FF = c->FF, MH = c->MH;
  Packer pk{cfg.dtype, {}};
  FPacker fp;
  size_t idx = 0;
  // band embedding: fold gamma_i * sqrt(W_i) into the projection, pad K to kpad_i
  c->emb_wband.resize(c->NB);
  c->emb_foff.resize(c->NB);
  std::vector<double> emb_bias, emb_frag;
  for (int i = 0; i < c->NB; ++i) {
    const std::vector<double>& g = W[idx++];
    const std::vector<double>& A = W[idx++];
    const std::vector<double>& b = W[idx++];
    const int Wi = bd.width[i], kp = c->kpad[i];
    const double r = std::sqrt((double)Wi);
    std::vector<double> m((size_t)D * kp, 0.0);
    for (int d = 0; d < D; ++d)
      for (int e = 0; e < Wi; ++e) m[(size_t)d * kp + e] = A[(size_t)d * Wi + e] * g[e] * r;
    if (c->use_embed) {
      c->emb_foff[i] = (int32_t)emb_frag.size();
      const std::vector<double> f = embed_stream(D, kp, m);
      emb_frag.insert(emb_frag.end(), f.begin(), f.end());
    } else {
      c->emb_wband[i] = pk.append(m);
    }
    emb_bias.insert(emb_bias.end(), b.begin(), b.end());
  }
  c->emb_b = fp.append(emb_bias);
  if (c->use_embed) c->emb_frag = pk.append(emb_frag);
  // transformers: attention gain (and the query scale dh^-1/2) folded into W_qkv and the gate
  // weights; feed-forward gain into W_1; output gain times sqrt(D) kept as a vector
  const double qscale = 1.0 / std::sqrt((double)c->DH);
  c->tw.resize(2 * cfg.depth);
  for (int t = 0; t < 2 * cfg.depth; ++t) {
    const auto& ga = W[idx++];
    const auto& wqkv = W[idx++];
    const auto& wg = W[idx++];
    const auto& bg = W[idx++];
    const auto& wout = W[idx++];
    const auto& gf = W[idx++];
    const auto& w1 = W[idx++];
    const auto& b1 = W[idx++];
    const auto& w2 = W[idx++];
    const auto& b2 = W[idx++];
    const auto& go = W[idx++];
    // 16-bit path: 64 more rows after q, k, v carry the gate projection (H rows, rest zero), so the
    // gates come out of the same product
    const int qrows = 3 * I + (cfg.dtype == MBR_F32 ? 0 : 64);
    std::vector<double> q((size_t)qrows * D, 0.0);
    for (int o = 0; o < 3 * I; ++o)
      for (int e = 0; e < D; ++e) q[(size_t)o * D + e] = wqkv[(size_t)o * D + e] * ga[e] * (o < I ? qscale : 1.0);
    if (cfg.dtype != MBR_F32)
      for (int hh = 0; hh < H; ++hh)
        for (int e = 0; e < D; ++e) q[(size_t)(3 * I + hh) * D + e] = wg[(size_t)hh * D + e] * ga[e];
    std::vector<double> g((size_t)H * D);
    for (int h = 0; h < H; ++h)
      for (int e = 0; e < D; ++e) g[(size_t)h * D + e] = wg[(size_t)h * D + e] * ga[e];
    std::vector<double> f1((size_t)FF * D);
    for (int o = 0; o < FF; ++o)
      for (int e = 0; e < D; ++e) f1[(size_t)o * D + e] = w1[(size_t)o * D + e] * gf[e];
    std::vector<double> gout(D);
    for (int e = 0; e < D; ++e) gout[e] = go[e] * std::sqrt((double)D);
    TransformerW& tw = c->tw[t];
    if (c->use_block) tw.bstream = pk.append(block_stream(D, I, FF, wout, f1, w2));
    tw.wqkv = pk.append(q);
    tw.wout = pk.append(wout);
    tw.w1 = pk.append(f1);
    tw.w2 = pk.append(w2);
    tw.wg = fp.append(g);
    tw.bg = fp.append(bg);
    tw.b1 = fp.append(b1);
    tw.b2 = fp.append(b2);
    tw.gout = fp.append(gout);
  }
  // mask head: per stem, per layer, bands in order; the last layer's value and gate rows
  // interleaved in blocks of glu_blk features so a GLU pair lands in one lane
  const int nl = cfg.mask_depth + 1;
  c->mw.resize(cfg.num_stems);
  for (int s = 0; s < cfg.num_stems; ++s) {
    MaskW& m = c->mw[s];
    m.wband.assign(nl, std::vector<size_t>(c->NB));
    m.bband.assign(nl, std::vector<size_t>(c->NB));
    for (int i = 0; i < c->NB; ++i) {
      for (int j = 0; j < nl; ++j) {
        const auto& w = W[idx++];
        const auto& b = W[idx++];
        if (j < nl - 1) {
          m.wband[j][i] = pk.append(w);
          m.bband[j][i] = fp.append(b);
        } else {
          const int Wi = bd.width[i], wp = c->wp[i], P = c->glu_blk;
          std::vector<double> r((size_t)2 * wp * MH, 0.0), rb((size_t)2 * wp, 0.0);
          for (int q = 0; q < wp / P; ++q)
            for (int k = 0; k < P; ++k) {
              const int e = P * q + k;
              if (e >= Wi) continue;
              for (int x = 0; x < MH; ++x) {
                r[(size_t)(2 * P * q + k) * MH + x] = w[(size_t)e * MH + x];
                r[(size_t)(2 * P * q + P + k) * MH + x] = w[(size_t)(Wi + e) * MH + x];
              }
              rb[2 * P * q + k] = b[e];
              rb[2 * P * q + P + k] = b[Wi + e];
            }
          m.wband[j][i] = pk.append(r);
          m.bband[j][i] = fp.append(rb);
        }
      }
    }
  }
  c->w_bytes = pk.bytes.size();
  c->f_bytes = fp.v.size() * 4;
  HIP_TRY(hipMalloc(&c->wdev, c->w_bytes));
  HIP_TRY(hipMemcpy(c->wdev, pk.bytes.data(), c->w_bytes, hipMemcpyHostToDevice));
  HIP_TRY(hipMalloc(&c->fdev, c->f_bytes));
  HIP_TRY(hipMemcpy(c->fdev, fp.v.data(), c->f_bytes, hipMemcpyHostToDevice));
  return MBR_OK;
}

int alloc_workspace(mbr_core* c) {
  const size_t esz = dtype_size(c->cfg.dtype);
  const size_t BT = (size_t)c->Bmax * c->T, NT = (size_t)c->NB * BT;
  size_t off = 0;
  auto place = [&](size_t bytes) {
    size_t o = (off + 255) / 256 * 256;
    off = o + bytes;
    return o;
  };
  const size_t attn_t = (size_t)c->NB * c->Bmax * c->H * c->Tp * c->DH * esz;
  const size_t attn_b = c->use_band ? 0 : BT * c->H * 64 * c->DH * esz;   // unused by the fused band kernel
  size_t oX = place(NT * c->D * 4), oXH = place(NT * c->D * esz), oG = place(NT * c->H * 4),
         oU = place(c->use_embed ? 0 : BT * c->kpad_total * esz), oqt = place(attn_t), okt = place(attn_t), ovt = place(attn_t),
         oqb = place(attn_b), okb = place(attn_b), ovb = place(attn_b), oO = place(NT * c->I * esz),
         oH1 = place(NT * std::max(c->FF, c->cfg.num_stems * c->MH) * esz),
         oH2 = place(NT * c->cfg.num_stems * c->MH * esz),
         oM = place((size_t)c->cfg.num_stems * BT * c->total * 4);
  size_t oSA = place(NT * kSsStride * 4), oSB = place(NT * kSsStride * 4), oSC = place(NT * kSsStride * 4);
  size_t oP = place(c->use_block ? block_part_bytes(c->D, (int64_t)NT, c->ncu) : 0);
  c->ws_bytes = off;
  hipError_t e = hipMalloc(&c->ws, off);
  if (e != hipSuccess) return fail(MBR_E_NOMEM, std::string("workspace hipMalloc: ") + hipGetErrorString(e));
  HIP_TRY(hipMemset(c->ws, 0, off));
  char* b = (char*)c->ws;
  c->X = (float*)(b + oX);
  c->XH = b + oXH;
  c->gates = (float*)(b + oG);
  c->U = b + oU;
  c->qt = b + oqt;
  c->kt = b + okt;
  c->vt = b + ovt;
  c->qb = b + oqb;
  c->kb = b + okb;
  c->vb = b + ovb;
  c->O = b + oO;
  c->H1 = b + oH1;
  c->H2 = b + oH2;
  c->Mglu = (float*)(b + oM);
  c->ssA = (float*)(b + oSA);
  c->ssB = (float*)(b + oSB);
  c->ssC = (float*)(b + oSC);
  c->part = (float*)(b + oP);
  return MBR_OK;
}

// ---------------------------------------------------------------------------------- forward
// Optional per-launch event timing (mbr_core_forward_profiled).
struct Prof {
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> marks;
  hipStream_t s;
  int begin(int kind) {
    hipEvent_t a, b;
    HIP_TRY(hipEventCreate(&a));
    HIP_TRY(hipEventCreate(&b));
    marks.push_back({kind, {a, b}});
    HIP_TRY(hipEventRecord(a, s));
    return MBR_OK;
  }
  int end() {
    HIP_TRY(hipEventRecord(marks.back().second.second, s));
    return MBR_OK;
  }
};

#define LAUNCH(kind, expr)                        \
  do {                                            \
    if (prof) { int r_ = prof->begin(kind); if (r_) return r_; } \
    HIP_TRY(expr);                                \
    if (prof) { int r_ = prof->end(); if (r_) return r_; } \
  } while (0)

hipError_t gemm(const GemmLaunch& L, int variant, hipStream_t s) {
  return L.dtype == DT_F32 ? launch_gemm(L, s) : launch_gemm2(L, variant, s);
}

int run_forward(mbr_core* c, const float* in, float* out, int batch, hipStream_t s, int stop_stage,
                Prof* prof = nullptr) {
  const mbr_config& cfg = c->cfg;
  const int dt = cfg.dtype;
  const int BT = batch * c->T;
  const int NT = c->NB * BT;
  const char* W = c->wdev;
  const size_t esz = dtype_size(dt);
  auto wptr = [&](size_t off) { return (const void*)(W + off * esz); };
  // 16-bit path: RMSNorms become row statistics written by the producing GEMM epilogues and row
  // scales applied by the consuming ones; the fp32 path runs explicit norm passes
  const bool fused = dt != MBR_F32;
  const int parts = c->D / 64;
  const float sqrtD = std::sqrt((float)c->D);

  if (c->use_embed) {
    // the band gather and the band embedding in one kernel: the gathered bands stay on the chip
    EmbedLaunch el{};
    el.dtype = dt;
    el.in = in;
    el.W = wptr(c->emb_frag);
    el.w_off = c->emb_woff;
    el.order = c->band_order;
    el.band_info = c->band_info;
    el.gather_pair = c->gather_pair;
    el.bias = c->fdev + c->emb_b;
    el.X = c->X;
    el.XH = c->XH;
    el.ss = c->ssB;     // x0's row sums of squares: the first attention's input norm
    el.num_bands = c->NB;
    el.batch = batch;
    el.frames = c->T;
    el.n_freqs = c->bands.n_freqs;
    el.channels = c->bands.channels;
    el.layout = cfg.io_layout;
    el.D = c->D;
    el.max_kpad = c->kpad_max;
    LAUNCH(MBR_K_EMBED, launch_embed(el, s));
  } else {
    GatherLaunch gl{dt, in, c->U, c->band_info, c->gather_pair, c->NB, batch, c->T, c->bands.n_freqs,
                    c->bands.channels, cfg.io_layout, c->kpad_max};
    LAUNCH(MBR_K_GATHER, launch_gather(gl, s));

    GemmLaunch ge{};
    ge.dtype = dt;
    ge.epi = EPI_EMBED;
    ge.A = c->U;
    ge.B = W;
    ge.C = c->X;
    ge.bias = c->fdev;
    ge.ldc = c->D;
    ge.M = BT;
    ge.groups = c->groups;
    ge.tiles = c->tiles + c->t_embed;
    ge.n_tiles = c->n_embed;
    if (fused) {
      ge.xh = c->XH;     // x0 in 16 bits and its row sums of squares: the first attention's input
      ge.ss1 = c->ssB;
      ge.ss_parts = parts;
    }
    LAUNCH(MBR_K_EMBED, gemm(ge, c->v_embed, s));
  }

  if (!fused) {
    NormLaunch nl{dt, 0, c->X, c->XH, nullptr, c->gates, c->fdev + c->tw[0].wg, c->fdev + c->tw[0].bg, NT, c->D, c->H};
    LAUNCH(MBR_K_NORM, launch_norm(nl, s));
  }
  if (stop_stage == 0) return MBR_OK;

  const int ntr = 2 * cfg.depth;
  for (int t = 0; t < ntr; ++t) {
    const TransformerW& tw = c->tw[t];
    const int axis = t & 1;
    if (axis == 1 && c->use_band) {
      // the band axis: q, k, v of one head for two frames, rotary, attention over the bands and
      // the gate, in one kernel (q, k, v stay on the chip)
      BandLaunch bd{};
      bd.dtype = dt;
      bd.XH = c->XH;
      bd.W = wptr(tw.wqkv);
      bd.gate_bias = c->fdev + tw.bg;
      bd.cos = c->cos_b;
      bd.sin = c->sin_b;
      if (!c->use_block) {   // XH carries the previous output, not yet normalised
        bd.rowss = c->ssB;
        bd.rs_mul = sqrtD;
      }
      bd.q_mul = 1.4426950408889634f;
      bd.O = c->O;
      bd.NB = c->NB;
      bd.BT = BT;
      bd.heads = c->H;
      bd.D = c->D;
      LAUNCH(MBR_K_BAND_ATTN, launch_band_attn(bd, s));
    } else {
    // q, k, v with rotary, scattered per axis
    GemmLaunch gq{};
    gq.dtype = dt;
    gq.epi = EPI_QKV;
    gq.A = c->XH;
    gq.B = wptr(tw.wqkv);
    gq.M = NT;
    gq.dense.N = 3 * c->I + (fused ? 64 : 0);
    gq.dense.K = c->D;
    if (fused) {
      if (t == 0 || !c->use_block) {   // otherwise XH arrives normalised
        gq.rowss = c->ssB;
        gq.ss_parts = parts;
        gq.rs_mul = sqrtD;
      }
      gq.gates = c->gates;
      gq.gate_bias = c->fdev + tw.bg;
    }
    gq.dense.lda = c->D;
    gq.dense.ldb = c->D;
    QkvArgs& qa = gq.qkv;
    qa.q = axis ? c->qb : c->qt;
    qa.k = axis ? c->kb : c->kt;
    qa.v = axis ? c->vb : c->vt;
    qa.cos = axis ? c->cos_b : c->cos_t;
    qa.sin = axis ? c->sin_b : c->sin_t;
    qa.axis = axis;
    qa.frames = c->T;
    qa.batch = batch;
    qa.heads = c->H;
    qa.dh = c->DH;
    qa.npad = axis ? 64 : c->Tp;
    // 16-bit path: q leaves the projection in log2 units for the exponentials of the attention
    qa.q_mul = fused ? 1.4426950408889634f : 1.0f;
    LAUNCH(MBR_K_QKV, gemm(gq, c->v_qkv, s));

    AttnLaunch al{};
    al.dtype = dt;
    al.axis = axis;
    al.q = qa.q;
    al.k = qa.k;
    al.v = qa.v;
    al.gates = c->gates;
    al.o = c->O;
    al.n = axis ? c->NB : c->T;
    al.npad = qa.npad;
    al.seqs = axis ? BT : c->NB * batch;
    al.heads = c->H;
    al.dh = c->DH;
    al.frames = c->T;
    al.batch = batch;
    // the 1/sqrt(dh) scale is folded into W_q; the 16-bit projection also applies log2(e)
    al.scale_log2 = fused ? 1.0f : 1.4426950408889634f;
    LAUNCH(axis ? MBR_K_ATTN_BAND : MBR_K_ATTN_TIME,
           (axis == 0 && dt != MBR_F32) ? launch_attention_time2(al, s) : launch_attention(al, s));
    }

    const bool last = t == ntr - 1;
    if (c->use_block) {
      // one 128-token group per compute unit at a time; the launch splits the hidden chunks of the
      // tokens after the last whole device pass over several blocks
      BlockLaunch bl{};
      bl.dtype = dt;
      bl.O = c->O;
      bl.stream = wptr(tw.bstream);
      bl.b1 = c->fdev + tw.b1;
      bl.b2 = c->fdev + tw.b2;
      bl.gout = c->fdev + tw.gout;
      bl.X = c->X;
      bl.XH = c->XH;
      bl.tokens = NT;
      bl.D = c->D;
      bl.I = c->I;
      bl.xh_norm = last ? 0 : 1;
      bl.ncu = c->ncu;
      bl.part = c->part;
      LAUNCH(MBR_K_BLOCK, launch_block(bl, s));
      if (stop_stage == 1 + t) return MBR_OK;   // X holds x after the output norm
      continue;
    }

    GemmLaunch go{};
    go.dtype = dt;
    go.epi = EPI_RESID;
    go.A = c->O;
    go.B = wptr(tw.wout);
    go.C = c->X;
    go.bias = nullptr;
    go.ldc = c->D;
    go.M = NT;
    go.dense.N = c->D;
    go.dense.K = c->I;
    go.dense.lda = c->I;
    go.dense.ldb = c->I;
    if (fused) {
      if (t > 0) {       // the previous Transformer's output norm, applied as the residual is read
        go.in_ss = c->ssA;
        go.in_gain = c->fdev + c->tw[t - 1].gout;
      }
      go.xh = c->XH;     // x in 16 bits and its row sums of squares: the feed-forward's input
      go.ss1 = c->ssC;
      go.ss_parts = parts;
    }
    LAUNCH(MBR_K_OUT_PROJ, gemm(go, c->v_out, s));

    if (!fused) {
      NormLaunch n0{dt, 0, c->X, c->XH, nullptr, nullptr, nullptr, nullptr, NT, c->D, c->H};
      LAUNCH(MBR_K_NORM, launch_norm(n0, s));
    }

    GemmLaunch g1{};
    g1.dtype = dt;
    g1.epi = EPI_GELU;
    g1.A = c->XH;
    g1.B = wptr(tw.w1);
    g1.C = c->H1;
    g1.bias = c->fdev;
    g1.dense.bias_off = (int64_t)tw.b1;
    g1.ldc = c->FF;
    g1.M = NT;
    g1.dense.N = c->FF;
    g1.dense.K = c->D;
    g1.dense.lda = c->D;
    g1.dense.ldb = c->D;
    if (fused) {
      g1.rowss = c->ssC;
      g1.ss_parts = parts;
      g1.rs_mul = sqrtD;
    }
    LAUNCH(MBR_K_FFN1, gemm(g1, c->v_ffn1, s));

    GemmLaunch g2{};
    g2.dtype = dt;
    g2.epi = EPI_FFN2;
    g2.A = c->H1;
    g2.B = wptr(tw.w2);
    g2.C = c->X;
    g2.bias = c->fdev;
    g2.dense.bias_off = (int64_t)tw.b2;
    g2.ldc = c->D;
    g2.M = NT;
    g2.dense.N = c->D;
    g2.dense.K = c->FF;
    g2.dense.lda = c->FF;
    g2.dense.ldb = c->FF;
    if (fused) {
      // x (before this Transformer's output norm) stays in X; x * gamma_out goes out in 16 bits with
      // the row sums of squares of x (ssA) and of x * gamma_out (ssB) for the consumers
      g2.xh = c->XH;
      g2.xh_gain = c->fdev + tw.gout;
      g2.xh_gmul = 1.0f / sqrtD;
      g2.ss1 = c->ssA;
      g2.ss2 = c->ssB;
      g2.ss_parts = parts;
    }
    LAUNCH(MBR_K_FFN2, gemm(g2, c->v_ffn2, s));

    if (!fused) {
      NormLaunch no{dt, last ? 2 : 1, c->X, c->XH, c->fdev + tw.gout, last ? nullptr : c->gates,
                    last ? nullptr : c->fdev + c->tw[t + 1].wg, last ? nullptr : c->fdev + c->tw[t + 1].bg,
                    NT, c->D, c->H};
      LAUNCH(MBR_K_NORM, launch_norm(no, s));
    }
    if (stop_stage == 1 + t) {
      if (fused) {       // taps show x after the output norm
        NormLaunch no{dt, 1, c->X, c->XH, c->fdev + tw.gout, nullptr, nullptr, nullptr, NT, c->D, c->H};
        HIP_TRY(launch_norm(no, s));
      }
      return MBR_OK;
    }
  }

  const int nlay = cfg.mask_depth + 1;
  const void* src = c->XH;
  for (int j = 0; j < nlay; ++j) {
    GemmLaunch gm{};
    gm.dtype = dt;
    gm.A = src;
    gm.B = W;
    gm.bias = c->fdev;
    gm.M = BT;
    gm.groups = c->groups;
    gm.tiles = c->tiles + c->t_mask[j];
    gm.n_tiles = c->n_mask[j];
    if (j < nlay - 1) {
      void* dst = (j % 2 == 0) ? c->H1 : c->H2;
      gm.epi = EPI_TANH;
      gm.C = dst;
      gm.ldc = c->MH;
      src = dst;
      if (fused && !c->use_block && j == 0) {   // the last Transformer's output norm, as a row scale
        gm.rowss = c->ssA;
        gm.ss_parts = parts;
        gm.rs_mul = sqrtD;
      }
    } else {
      gm.epi = EPI_GLU;
      gm.C = c->Mglu;
      gm.glu_total = c->total;
      gm.glu_frames = c->T;
    }
    LAUNCH(j < nlay - 1 ? MBR_K_MASK_HIDDEN : MBR_K_MASK_GLU, gemm(gm, j < nlay - 1 ? c->v_mask : c->v_glu, s));
  }
  if (stop_stage == 1000) return MBR_OK;

  AverageLaunch av{c->Mglu, out, c->inv_slot, c->inv_weight, batch, cfg.num_stems, c->total, c->T,
                   c->bands.n_freqs, c->bands.channels, cfg.io_layout};
  LAUNCH(MBR_K_AVERAGE, launch_average(av, s));
  return MBR_OK;
}

}  // namespace

// ====================================================================================== C ABI
extern "C" {

const char* mbr_last_error(void) { return g_err.c_str(); }

int mbr_core_weight_count(const mbr_config* cfg) {
  if (!cfg) return fail(MBR_E_ARG, "cfg is NULL");
  Bands b;
  std::string err;
  int rc = build_bands(*cfg, &b, &err);
  if (rc) return fail(rc, err);
  return (int)inventory(*cfg, b).size();
}

int mbr_core_weight_info(const mbr_config* cfg, int index, int* ndim, int64_t dims[2], int* kind) {
  if (!cfg || !ndim || !dims || !kind) return fail(MBR_E_ARG, "NULL argument");
  Bands b;
  std::string err;
  int rc = build_bands(*cfg, &b, &err);
  if (rc) return fail(rc, err);
  auto inv = inventory(*cfg, b);
  if (index < 0 || index >= (int)inv.size()) return fail(MBR_E_ARG, "weight index out of range");
  *ndim = inv[index].ndim;
  dims[0] = inv[index].rows;
  dims[1] = inv[index].cols;
  *kind = inv[index].kind;
  return MBR_OK;
}

int mbr_core_table_sizes(const mbr_config* cfg, int32_t* num_bands, int32_t* total_width, int32_t* n_freqs) {
  if (!cfg) return fail(MBR_E_ARG, "cfg is NULL");
  Bands b;
  std::string err;
  int rc = build_bands(*cfg, &b, &err);
  if (rc) return fail(rc, err);
  if (num_bands) *num_bands = b.num_bands();
  if (total_width) *total_width = b.total_width();
  if (n_freqs) *n_freqs = b.n_freqs;
  return MBR_OK;
}

int mbr_core_tables(const mbr_config* cfg, int32_t* band_bins, int32_t* band_offset, int32_t* gather_pair,
                    int32_t* inv_slot, float* inv_weight, int32_t* bin_count) {
  if (!cfg) return fail(MBR_E_ARG, "cfg is NULL");
  Bands b;
  std::string err;
  int rc = build_bands(*cfg, &b, &err);
  if (rc) return fail(rc, err);
  for (int i = 0; i < b.num_bands(); ++i) {
    if (band_bins) band_bins[i] = (int32_t)b.bins[i].size();
  }
  if (band_offset)
    for (int i = 0; i <= b.num_bands(); ++i) band_offset[i] = b.offset[i];
  if (gather_pair) std::memcpy(gather_pair, b.gather_pair.data(), b.gather_pair.size() * 4);
  if (inv_slot) std::memcpy(inv_slot, b.inv_slot.data(), b.inv_slot.size() * 4);
  if (inv_weight) std::memcpy(inv_weight, b.inv_weight.data(), b.inv_weight.size() * 4);
  if (bin_count) std::memcpy(bin_count, b.count.data(), b.count.size() * 4);
  return MBR_OK;
}

int mbr_core_create(const mbr_config* cfg, const void* const* weights, int n_weights, mbr_core** out) {
  if (!out) return fail(MBR_E_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg || !weights) return fail(MBR_E_ARG, "NULL argument");
  mbr_core* c = new (std::nothrow) mbr_core();
  if (!c) return fail(MBR_E_NOMEM, "host allocation failed");
  c->cfg = *cfg;
  c->cfg.band_bins = nullptr;   // the caller's table is read here only; the bands keep it
  std::string err;
  int rc = build_bands(*cfg, &c->bands, &err);
  if (rc) {
    delete c;
    return fail(rc, err);
  }
  if (cfg->num_bands > 64) {
    delete c;
    return fail(MBR_E_CONFIG, "invalid config: the band-axis attention supports at most 64 bands");
  }
  rc = check_device(&c->device, &c->ncu);
  if (rc) {
    delete c;
    return rc;
  }
  auto inv = inventory(*cfg, c->bands);
  if (n_weights != (int)inv.size()) {
    delete c;
    return fail(MBR_E_ARG, "expected " + std::to_string(inv.size()) + " weight tensors, got " + std::to_string(n_weights));
  }
  c->NB = cfg->num_bands;
  c->D = cfg->dim;
  c->H = cfg->heads;
  c->DH = cfg->dim_head;
  c->I = c->H * c->DH;
  c->FF = cfg->ff_mult * c->D;
  c->MH = cfg->mask_hidden_mult * c->D;
  c->T = cfg->frames;
  c->Tp = round_up(c->T, 128);
  c->Bmax = cfg->max_batch;
  c->total = c->bands.total_width();
  const int kstep = cfg->dtype == MBR_F32 ? 16 : 32;
  c->glu_blk = cfg->dtype == MBR_F32 ? 16 : 32;
  // tile configuration of the 16-bit GEMM per launch kind, from a sweep on MI355X at the core's
  // shapes: 256 x 128 tiles of 64 x 64 waves, 3 stages, was the fastest for every product
  c->v_qkv = 4;
  c->v_ffn1 = 4;
  c->v_ffn2 = 4;
  c->v_out = 4;
  c->v_mask = 4;
  c->v_glu = 2;
  c->v_embed = 4;
  c->use_block = block_supported(cfg->dtype, c->D, c->I, c->FF);
  c->use_band = band_attn_supported(cfg->dtype, c->NB, c->H, c->DH, c->D);
  c->kpad.resize(c->NB);
  c->kcol.resize(c->NB);
  c->wp.resize(c->NB);
  int col = 0;
  for (int i = 0; i < c->NB; ++i) {
    c->kpad[i] = round_up(c->bands.width[i], kstep);
    c->kcol[i] = col;
    col += c->kpad[i];
    c->kpad_max = std::max(c->kpad_max, c->kpad[i]);
    c->wp[i] = round_up(c->bands.width[i], c->glu_blk);
  }
  c->kpad_total = col;
  c->use_embed = embed_fused_supported(cfg->dtype, c->D, c->kpad_max);
  // read the caller's weights
  std::vector<std::vector<double>> W(inv.size());
  const size_t esz = dtype_size(cfg->dtype);
  for (size_t i = 0; i < inv.size(); ++i) {
    if (!weights[i]) {
      delete c;
      return fail(MBR_E_ARG, "weight " + std::to_string(i) + " (" + inv[i].name + ") is NULL");
    }
    const size_t n = (size_t)inv[i].rows * inv[i].cols;
    std::vector<char> raw(n * esz);
    hipError_t e = hipMemcpy(raw.data(), weights[i], n * esz, hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
      delete c;
      return fail(MBR_E_HIP, "copying weight " + inv[i].name + ": " + hipGetErrorString(e));
    }
    W[i] = to_double(raw, cfg->dtype, n);
  }
  rc = repack_weights(c, W);
  if (!rc) rc = setup_tables_and_groups(c);
  if (!rc) rc = alloc_workspace(c);
  if (!rc) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = fail(MBR_E_HIP, std::string("hipDeviceSynchronize: ") + hipGetErrorString(e));
  }
  if (rc) {
    mbr_core_destroy(c);
    return rc;
  }
  *out = c;
  return MBR_OK;
}

int mbr_core_forward(mbr_core* c, const float* in, float* out, int batch, hipStream_t stream) {
  if (!c || !in || !out) return fail(MBR_E_ARG, "NULL argument");
  if (batch < 1 || batch > c->Bmax) return fail(MBR_E_ARG, "batch out of range 1..max_batch");
  return run_forward(c, in, out, batch, stream, -1);
}

int64_t mbr_core_debug_size(const mbr_core* c, int batch, int stage) {
  if (!c || batch < 1 || batch > c->Bmax) return fail(MBR_E_ARG, "bad core or batch");
  const int64_t BT = (int64_t)batch * c->T;
  if (stage >= 0 && stage <= 2 * c->cfg.depth) return (int64_t)c->NB * BT * c->D;
  if (stage == 1000) return BT * c->total;
  return fail(MBR_E_ARG, "unknown stage");
}

int mbr_core_forward_debug(mbr_core* c, const float* in, int batch, int stage, float* out, hipStream_t stream) {
  if (!c || !in || !out) return fail(MBR_E_ARG, "NULL argument");
  int64_t n = mbr_core_debug_size(c, batch, stage);
  if (n < 0) return (int)n;
  int rc = run_forward(c, in, nullptr, batch, stream, stage);
  if (rc) return rc;
  const void* src = stage == 1000 ? (const void*)c->Mglu : (const void*)c->X;
  HIP_TRY(hipMemcpyAsync(out, src, (size_t)n * 4, hipMemcpyDeviceToDevice, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  return MBR_OK;
}

int mbr_core_forward_profiled(mbr_core* c, const float* in, float* out, int batch, hipStream_t stream,
                              double* ms_per_kind, int32_t* launches_per_kind) {
  if (!c || !in || !out || !ms_per_kind || !launches_per_kind) return fail(MBR_E_ARG, "NULL argument");
  if (batch < 1 || batch > c->Bmax) return fail(MBR_E_ARG, "batch out of range 1..max_batch");
  Prof p;
  p.s = stream;
  int rc = run_forward(c, in, out, batch, stream, -1, &p);
  hipError_t e = hipStreamSynchronize(stream);
  for (int k = 0; k < MBR_K_COUNT; ++k) {
    ms_per_kind[k] = 0.0;
    launches_per_kind[k] = 0;
  }
  for (auto& m : p.marks) {
    float ms = 0.f;
    if (!rc && e == hipSuccess && hipEventElapsedTime(&ms, m.second.first, m.second.second) == hipSuccess) {
      ms_per_kind[m.first] += ms;
      launches_per_kind[m.first] += 1;
    }
    (void)hipEventDestroy(m.second.first);
    (void)hipEventDestroy(m.second.second);
  }
  if (rc) return rc;
  if (e != hipSuccess) return fail(MBR_E_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
  return MBR_OK;
}

int mbr_k_gemm_variants(void) { return gemm2_variants(); }

int mbr_k_gelu(const float* x, float* y, int n, hipStream_t stream) {
  if (!x || !y || n < 0) return fail(MBR_E_ARG, "bad argument");
  HIP_TRY(launch_gelu(x, y, n, stream));
  return MBR_OK;
}

int mbr_k_gemm(int dtype, const void* a, const void* b, const float* bias, void* cmat, int M, int N, int K,
               int variant, int out16, hipStream_t stream) {
  if (!a || !b || !cmat) return fail(MBR_E_ARG, "NULL argument");
  if (M < 1 || N < 1 || K < 1 || N % 64 || K % (dtype == MBR_F32 ? 16 : 32))
    return fail(MBR_E_ARG, "mbr_k_gemm needs N % 64 == 0 and K a multiple of the K step");
  if (dtype != MBR_F32 && (variant < 0 || variant >= gemm2_variants())) return fail(MBR_E_ARG, "unknown variant");
  if (dtype != MBR_F32 && dtype != MBR_F16 && dtype != MBR_BF16) return fail(MBR_E_ARG, "unknown dtype");
  GemmLaunch L{};
  if (out16 && dtype == MBR_F32) return fail(MBR_E_ARG, "16-bit output needs a 16-bit dtype");
  L.dtype = dtype;
  L.epi = out16 ? EPI_STORE16 : EPI_EMBED;
  L.A = a;
  L.B = b;
  L.C = cmat;
  L.bias = bias;
  L.ldc = N;
  L.M = M;
  L.dense.N = N;
  L.dense.K = K;
  L.dense.lda = K;
  L.dense.ldb = K;
  HIP_TRY(gemm(L, variant, stream));
  return MBR_OK;
}

int mbr_attention(int dtype, const void* q, const void* k, const void* vt, const float* gates, void* o, int seqs,
                  int heads, int n, int npad, int dqk, int dv, float scale, hipStream_t stream) {
  if (!q || !k || !vt || !o) return fail(MBR_E_ARG, "NULL argument");
  if (dtype != MBR_F16 && dtype != MBR_BF16) return fail(MBR_E_ARG, "attention: dtype must be MBR_F16 or MBR_BF16");
  if (seqs < 1 || heads < 1 || n < 1 || npad < n || npad % 128)
    return fail(MBR_E_ARG, "attention: seqs, heads >= 1, 1 <= n <= npad, npad a multiple of 128");
  if (!attention_time2_supported(dqk, dv))
    return fail(MBR_E_ARG, "attention: (dqk, dv) must be (32, 32), (64, 64) or (128, 64)");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(MBR_E_ARG, "attention: scale must be positive and finite");
  if ((int64_t)seqs * heads * (npad / 128) > INT32_MAX || (int64_t)npad * dqk * 2 > INT32_MAX)
    return fail(MBR_E_ARG, "attention: sizes too large");
  AttnLaunch al{};
  al.dtype = dtype;
  al.axis = 0;
  al.q = q;
  al.k = k;
  al.v = vt;
  al.gates = gates;
  al.o = o;
  al.n = n;
  al.npad = npad;
  al.seqs = seqs;
  al.heads = heads;
  al.dh = dqk;
  al.dv = dv;
  al.frames = n;
  al.batch = 1;
  al.scale_log2 = 1.0f;
  al.q_mul = scale * 1.4426950408889634f;   // scores in log2 units for the exponentials
  HIP_TRY(launch_attention_time2(al, stream));
  return MBR_OK;
}

int64_t mbr_core_device_bytes(const mbr_core* c) {
  if (!c) return 0;
  return (int64_t)(c->w_bytes + c->f_bytes + c->ws_bytes);
}

// ---- around the core ------------------------------------------------------------------
int mbr_stft(const float* wave, int channels, int64_t length, int n_fft, int hop, float* spec, hipStream_t stream) {
  if (!wave || !spec) return fail(MBR_E_ARG, "NULL argument");
  if (channels < 1 || length < 2 || !stft_supported(n_fft) || hop < 1 || hop > n_fft / 2)
    return fail(MBR_E_ARG, "stft: channels >= 1, length >= 2, n_fft a power of two in 16..4096, 1 <= hop <= n_fft/2");
  StftGeom G{};
  G.wave = wave;
  G.S = channels;
  G.n_fft = n_fft;
  G.hop = hop;
  G.T = (int32_t)(1 + length / hop);
  G.no_fade = 1;
  G.L = G.Lp = G.chunk = G.stride = length;
  HIP_TRY(launch_stft(G, 1, spec, stream));
  return MBR_OK;
}

int64_t mbr_istft_workspace_size(int channels, int n_fft, int frames, int stems) {
  if (channels < 1 || frames < 1 || stems < 1 || !stft_supported(n_fft)) return fail(MBR_E_ARG, "bad sizes");
  return (int64_t)stems * channels * frames * n_fft * 4;
}

int mbr_istft_masked(const float* spec, const float* masks, int stems, int channels, int64_t length, int n_fft,
                     int hop, void* workspace, float* out, hipStream_t stream) {
  if (!spec || !masks || !workspace || !out) return fail(MBR_E_ARG, "NULL argument");
  if (channels < 1 || stems < 1 || length < 2 || !stft_supported(n_fft) || hop < 1 || hop > n_fft / 2)
    return fail(MBR_E_ARG, "istft: bad sizes");
  StftGeom G{};
  G.S = channels;
  G.n_fft = n_fft;
  G.hop = hop;
  G.T = (int32_t)(1 + length / hop);
  G.no_fade = 1;
  G.L = G.Lp = G.chunk = G.stride = length;
  float* frames = (float*)workspace;
  HIP_TRY(launch_istft_frames(G, 1, spec, masks, stems, frames, stream));
  HIP_TRY(launch_fill0(out, (int64_t)stems * channels * length, stream));
  HIP_TRY(launch_ola(G, frames, stems, 1, 0, length, out, nullptr, stream));
  return MBR_OK;
}

int mbr_istft_masked_noalloc(const float* spec, const float* masks, int stems, int channels, int64_t length,
                             int n_fft, int hop, float* out, hipStream_t stream) {
  if (!spec || !masks || !out) return fail(MBR_E_ARG, "NULL argument");
  if (channels < 1 || stems < 1 || length < 2 || !stft_supported(n_fft) || hop < 1 || hop > n_fft / 2)
    return fail(MBR_E_ARG, "istft: bad sizes");
  const int64_t T = 1 + length / hop;
  const int64_t need = (int64_t)stems * channels * T * n_fft * 4;
  if (need > MBR_ISTFT_NOALLOC_MAX_BYTES)
    return fail(MBR_E_ARG, "istft (no allocation): stems * channels * frames * n_fft * 4 = " + std::to_string(need) +
                               " bytes exceeds the static buffer of " + std::to_string((int64_t)MBR_ISTFT_NOALLOC_MAX_BYTES));
  static_assert(MBR_ISTFT_NOALLOC_MAX_BYTES == kIstftNoallocBytes, "header and library agree on the buffer size");
  void* frames = nullptr;
  HIP_TRY(istft_noalloc_scratch(&frames));
  StftGeom G{};
  G.S = channels;
  G.n_fft = n_fft;
  G.hop = hop;
  G.T = (int32_t)T;
  G.no_fade = 1;
  G.L = G.Lp = G.chunk = G.stride = length;
  // every element of the frames this call reads is written by its own istft_frames launch first
  HIP_TRY(launch_istft_frames(G, 1, spec, masks, stems, (float*)frames, stream));
  HIP_TRY(launch_fill0(out, (int64_t)stems * channels * length, stream));
  HIP_TRY(launch_ola(G, (const float*)frames, stems, 1, 0, length, out, nullptr, stream));
  return MBR_OK;
}

namespace {
struct SepPlan {
  StftGeom G{};
  int n_chunks = 0, group = 0, stems = 0;
  size_t o_spec = 0, o_masks = 0, o_frames = 0, o_out = 0, o_cnt = 0, bytes = 0;
};

int plan_separation(const mbr_core* c, int64_t length, int hop, int64_t stride, SepPlan* P) {
  const mbr_config& cfg = c->cfg;
  if (cfg.io_layout != MBR_IO_FS_T_C) return fail(MBR_E_ARG, "separate: the core must use MBR_IO_FS_T_C");
  if (!stft_supported(cfg.n_fft) || hop < 1 || hop > cfg.n_fft / 2) return fail(MBR_E_ARG, "separate: bad hop / n_fft");
  const int64_t chunk = (int64_t)(c->T - 1) * hop;
  if (chunk < 20 || length < 2) return fail(MBR_E_ARG, "separate: the core's frames give a chunk of under 20 samples");
  StftGeom& G = P->G;
  G.S = c->bands.channels;
  G.n_fft = cfg.n_fft;
  G.hop = hop;
  G.T = c->T;
  G.chunk = chunk;
  if (stride < 0 || stride > chunk - chunk / 10)
    return fail(MBR_E_ARG, "separate: the stride must be 0 (0.9 chunk) or 1 .. chunk - chunk/10 samples (chunk = " +
                               std::to_string(chunk) + ")");
  G.stride = stride > 0 ? stride : (int64_t)(chunk * 0.9);
  const int64_t border = chunk - G.stride;
  G.pad = length > 2 * border ? border : 0;
  G.L = length;
  G.Lp = length + 2 * G.pad;
  P->n_chunks = (int)((G.Lp + G.stride - 1) / G.stride);
  P->group = std::min(P->n_chunks, c->Bmax);
  P->stems = cfg.num_stems;
  const int64_t F = cfg.n_fft / 2 + 1, spec1 = F * G.S * G.T * 2 * 4;
  size_t off = 0;
  auto place = [&](size_t b) {
    size_t o = (off + 255) / 256 * 256;
    off = o + b;
    return o;
  };
  P->o_spec = place((size_t)P->group * spec1);
  P->o_masks = place((size_t)P->group * P->stems * spec1);
  P->o_frames = place((size_t)P->group * P->stems * G.S * G.T * cfg.n_fft * 4);
  P->o_out = place((size_t)P->stems * G.S * G.Lp * 4);
  P->o_cnt = place((size_t)G.Lp * 4);
  P->bytes = off;
  return MBR_OK;
}
}  // namespace

int64_t mbr_separate_workspace_size_strided(const mbr_core* c, int64_t length, int hop, int64_t stride) {
  if (!c) return fail(MBR_E_ARG, "NULL core");
  SepPlan P;
  int rc = plan_separation(c, length, hop, stride, &P);
  return rc ? rc : (int64_t)P.bytes;
}

int64_t mbr_separate_workspace_size(const mbr_core* c, int64_t length, int hop) {
  return mbr_separate_workspace_size_strided(c, length, hop, 0);
}

int mbr_separate_strided(mbr_core* c, const float* wave, int64_t length, int hop, int64_t stride, void* workspace,
                         float* out, hipStream_t stream) {
  if (!c || !wave || !workspace || !out) return fail(MBR_E_ARG, "NULL argument");
  SepPlan P;
  int rc = plan_separation(c, length, hop, stride, &P);
  if (rc) return rc;
  StftGeom& G = P.G;
  G.wave = wave;
  char* ws = (char*)workspace;
  float *spec = (float*)(ws + P.o_spec), *masks = (float*)(ws + P.o_masks), *frames = (float*)(ws + P.o_frames),
        *acc = (float*)(ws + P.o_out), *cnt = (float*)(ws + P.o_cnt);
  HIP_TRY(launch_fill0(acc, (int64_t)P.stems * G.S * G.Lp, stream));
  HIP_TRY(launch_fill0(cnt, G.Lp, stream));
  for (int c0 = 0; c0 < P.n_chunks; c0 += P.group) {
    const int g = std::min(P.group, P.n_chunks - c0);
    G.chunk0 = c0;
    HIP_TRY(launch_stft(G, g, spec, stream));
    rc = run_forward(c, spec, masks, g, stream, -1);
    if (rc) return rc;
    HIP_TRY(launch_istft_frames(G, g, spec, masks, P.stems, frames, stream));
    const int64_t lo = (int64_t)c0 * G.stride, hi = std::min(G.Lp, (int64_t)(c0 + g - 1) * G.stride + G.chunk);
    HIP_TRY(launch_ola(G, frames, P.stems, g, lo, hi, acc, cnt, stream));
  }
  HIP_TRY(launch_finish(G, P.stems, acc, cnt, out, stream));
  return MBR_OK;
}

int mbr_separate(mbr_core* c, const float* wave, int64_t length, int hop, void* workspace, float* out,
                 hipStream_t stream) {
  return mbr_separate_strided(c, wave, length, hop, 0, workspace, out, stream);
}

void mbr_core_destroy(mbr_core* c) {
  if (!c) return;
  if (c->wdev) (void)hipFree(c->wdev);
  if (c->fdev) (void)hipFree(c->fdev);
  if (c->ws) (void)hipFree(c->ws);
  if (c->tables_dev) (void)hipFree(c->tables_dev);
  delete c;
}

}  // extern "C"
