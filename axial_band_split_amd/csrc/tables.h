// Host-side tables of the core: mel band membership, gather / inverse index, rotary tables,
// weight inventory.  Built once at mbr_core_create (and by the table query entry points).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mbr_core.h"

namespace mbr {

struct Bands {
  int n_freqs = 0;                    // F = n_fft/2 + 1
  int channels = 0;                   // S
  std::vector<std::vector<int>> bins; // per band, ascending
  std::vector<int> width;             // W_i = 2*S*|bins_i|
  std::vector<int> offset;            // feature offset of band i (size NB + 1)
  std::vector<int> gather_pair;       // slot -> pair (bin*S + s), slots of all bands in order
  std::vector<int> inv_slot;          // [F*S][2]: slots holding pair p, -1 if none
  std::vector<float> inv_weight;      // [F*S]: 1 / count(bin)
  std::vector<int> count;             // [F]
  int total_width() const { return offset.back(); }
  int num_bands() const { return (int)bins.size(); }
};

// Returns MBR_OK or MBR_E_CONFIG with `err` set.
int build_bands(const mbr_config& cfg, Bands* out, std::string* err);

struct WeightInfo {
  std::string name;
  int ndim;
  int64_t rows, cols;  // cols = 1 for vectors
  int kind;
};

int validate_config(const mbr_config& cfg, std::string* err);
// Inventory in canonical order; requires the bands of cfg.
std::vector<WeightInfo> inventory(const mbr_config& cfg, const Bands& bands);

// Rotary cos / sin tables [n][dh/2] for positions 0..n-1, angles evaluated in double and rounded
// once to float.
void rope_tables(int n, int dh, std::vector<float>* cos_t, std::vector<float>* sin_t);

}  // namespace mbr
