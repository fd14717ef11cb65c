// Host-side table code of the core (csrc/tables.cpp) built on its own with the address and
// undefined-behaviour sanitizers (by test_host_sanitized.py): builds the tables of one configuration
// given on the command line and prints them for comparison with the shipped library's.
//   host_tables_driver sample_rate n_fft channels num_bands dim depth heads dim_head ff_mult
//                      mask_hidden_mult mask_depth num_stems max_batch frames dtype io_layout zero_dc
//                      [bins of band 0 .. bins of band num_bands-1]
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tables.h"

int main(int argc, char** argv) {
  if (argc < 18) {
    std::fprintf(stderr, "usage: %s <17 config fields> [band bins...]\n", argv[0]);
    return 2;
  }
  mbr_config c;
  std::memset(&c, 0, sizeof c);
  int32_t* f[] = {&c.sample_rate, &c.n_fft, &c.audio_channels, &c.num_bands, &c.dim, &c.depth, &c.heads,
                  &c.dim_head, &c.ff_mult, &c.mask_hidden_mult, &c.mask_depth, &c.num_stems, &c.max_batch,
                  &c.frames, &c.dtype, &c.io_layout, &c.zero_dc};
  for (int i = 0; i < 17; ++i) *f[i] = std::atoi(argv[1 + i]);
  std::vector<int32_t> bins;
  for (int i = 18; i < argc; ++i) bins.push_back(std::atoi(argv[i]));
  c.band_bins = bins.empty() ? nullptr : bins.data();

  std::string err;
  int rc = mbr::validate_config(c, &err);
  mbr::Bands b;
  if (rc == 0) rc = mbr::build_bands(c, &b, &err);
  std::printf("rc %d\n", rc);
  if (rc != 0) return 0;
  auto row = [](const char* key, const std::vector<int>& v) {
    std::printf("%s", key);
    for (int x : v) std::printf(" %d", x);
    std::printf("\n");
  };
  std::vector<int> nb;
  for (const auto& bb : b.bins) nb.push_back((int)bb.size());
  row("band_bins", nb);
  row("band_offset", b.offset);
  row("gather_pair", b.gather_pair);
  row("inv_slot", b.inv_slot);
  row("bin_count", b.count);
  std::vector<int> wbits;
  for (float w : b.inv_weight) {
    uint32_t u;
    std::memcpy(&u, &w, 4);
    wbits.push_back((int)u);
  }
  row("inv_weight_bits", wbits);
  std::vector<int> shapes;
  for (const auto& wi : mbr::inventory(c, b)) {
    shapes.push_back((int)wi.rows);
    shapes.push_back((int)wi.cols);
  }
  row("inventory", shapes);
  for (int n : {c.frames, 64}) {
    std::vector<float> cs, sn;
    mbr::rope_tables(n, c.dim_head, &cs, &sn);
    double s = 0.0;
    for (size_t i = 0; i < cs.size(); ++i) s += (double)cs[i] * (i % 7 + 1) + (double)sn[i] * (i % 5 + 1);
    std::printf("rope %d %zu %.17g\n", n, cs.size(), s);
  }
  return 0;
}
