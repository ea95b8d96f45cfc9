// Host-only driver of the library's plan (plan.cpp), built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by test_plan_sanitized.py.
//
// Reads descriptor cases from a binary file: per case the four int32 shape
// fields, the raw bytes of one relpos_desc (its explicit_rows pointer is
// replaced here), an int32 count of explicit rows and the rows.  Prints one
// line per case: the return code, then (on success) the saturation radius,
// the expanded rows and the buffer sizes the exported relpos_plan_sizes
// reports for the same plan.
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "plan.hpp"

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s cases.bin\n", argv[0]);
    return 2;
  }
  std::FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  for (;;) {
    int32_t shp[4];
    if (std::fread(shp, sizeof shp, 1, f) != 1) break;
    relpos_desc d;
    if (std::fread(&d, sizeof d, 1, f) != 1) return 3;
    int32_t nrows = 0;
    if (std::fread(&nrows, sizeof nrows, 1, f) != 1 || nrows < 0) return 3;
    std::vector<int32_t> rows(static_cast<size_t>(nrows));
    if (nrows > 0 && std::fread(rows.data(), sizeof(int32_t), rows.size(), f) != rows.size())
      return 3;
    d.map.explicit_rows = nrows > 0 ? rows.data() : nullptr;
    relpos_shape sh{shp[0], shp[1], shp[2], shp[3]};
    relpos::Plan p;
    std::string detail;
    const int rc = relpos::make_plan(&d, &sh, p, detail);
    if (rc != RELPOS_OK) {
      std::printf("%d\n", rc);
      continue;
    }
    std::printf("%d %d %d %zu %zu %zu %zu\n", rc, p.delta, p.S, p.z_bytes, p.ws_fwd_end,
                p.ws_bwd_end, static_cast<size_t>(p.NG));
  }
  std::fclose(f);
  return 0;
}
