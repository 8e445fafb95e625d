// Host check: the kernels' block addressing (block_position(), and its split
// into a uniform block part and a per-row part) agrees with row_position() /
// key_position() for every kernel row and key of many geometries.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../factorized_sparse_self_amd/csrc/st_internal.hpp"
#include "../../include/st.h"

using namespace st;

int main() {
  const int patterns[] = {ST_STRIDED, ST_FIXED, ST_FIXED_R1, ST_DENSE, ST_STRIDED_UNION, ST_FIXED_UNION};
  const int Ts[] = {1, 5, 63, 64, 65, 200, 250, 1000, 1024, 4099};
  const int ls[] = {1, 2, 3, 7, 16, 20, 64, 96, 128, 300};
  long checked = 0;
  for (int pattern : patterns)
    for (int T : Ts)
      for (int l : ls)
        for (int c = 1; c <= l && c <= 9; c += (c < 4 ? 1 : 4)) {
          // the default summary set (last c offsets) and a spread one, o*l/c
          std::vector<int32_t> spread(c);
          for (int o = 0; o < c; ++o) spread[o] = (int32_t)((long)o * l / c);
          const bool fixed = pattern == ST_FIXED || pattern == ST_FIXED_R1 || pattern == ST_FIXED_UNION;
          for (int variant = 0; variant < (fixed ? 2 : 1); ++variant)
          for (int kind = 0; kind < 2; ++kind) {
            Geometry g;
            make_geometry(pattern, kind, T, l, c, variant ? spread.data() : nullptr, &g);
            // a position is a kernel key exactly when position_is_key says so
            {
              std::vector<char> is_key(T, 0);
              for (int K = 0; K < g.n_keys; ++K) {
                const int p = key_position(g, K);
                if (p >= 0) is_key[p] = 1;
              }
              for (int t = 0; t < T; ++t)
                if ((bool)is_key[t] != position_is_key(g, t)) {
                  std::printf("key set mismatch p%d T%d l%d c%d kind%d var%d t%d\n", pattern, T, l, c, kind,
                              variant, t);
                  return 1;
                }
            }
            const int nrb = (g.n_rows + kBlock - 1) / kBlock, nkb = (g.n_keys + kBlock - 1) / kBlock;
            for (int b = 0; b < nrb; ++b)
              for (int i = 0; i < kBlock; ++i) {
                const int want = row_position(g, b * kBlock + i);
                const int got = block_position(g, false, b, i);
                if (want != got) {
                  std::printf("row mismatch p%d T%d l%d c%d kind%d R%d: %d vs %d\n", pattern, T, l, c, kind,
                              b * kBlock + i, got, want);
                  return 1;
                }
                ++checked;
              }
            for (int keys = 0; keys < 2; ++keys) {
              if (!split_position_ok(g, keys)) continue;
              const int nb_ = keys ? nkb : nrb;
              for (int b = 0; b < nb_; ++b) {
                const BlockPart bp = block_part(g, keys, b);
                for (int i = 0; i < kBlock; ++i) {
                  const int q = (residue_major(g) && i >= bp.split ? bp.base2 : bp.base) + row_part(g, keys, i).off;
                  const int got = (i < bp.limit && q < g.T) ? q : -1;
                  const int want = block_position(g, keys, b, i);
                  if (want != got) {
                    std::printf("split mismatch p%d T%d l%d c%d kind%d keys%d blk%d i%d: %d vs %d\n", pattern, T,
                                l, c, kind, keys, b, i, got, want);
                    return 1;
                  }
                  ++checked;
                }
              }
            }
            for (int b = 0; b < nkb; ++b)
              for (int i = 0; i < kBlock; ++i) {
                const int want = key_position(g, b * kBlock + i);
                const int got = block_position(g, true, b, i);
                if (want != got) {
                  std::printf("key mismatch p%d T%d l%d c%d kind%d K%d: %d vs %d\n", pattern, T, l, c, kind,
                              b * kBlock + i, got, want);
                  return 1;
                }
                ++checked;
              }
          }
          if (pattern != ST_FIXED && pattern != ST_FIXED_R1 && pattern != ST_FIXED_UNION) break;
        }
  std::printf("ok %ld\n", checked);
  return 0;
}
