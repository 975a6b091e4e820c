// Host-side check of the latent-grid cube helpers in csrc/common.hpp: prints, for
// every cube of the grid given on the command line, its token count and tokens.
#include "common.hpp"

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  vdit::CubeGeom g{};
  g.on = 1;
  g.t = std::atoi(argv[1]);
  g.h = std::atoi(argv[2]);
  g.w = std::atoi(argv[3]);
  g.nct = (g.t + 3) / 4;
  g.ncy = (g.h + 3) / 4;
  g.ncx = (g.w + 3) / 4;
  g.n = g.nct * g.ncy * g.ncx;
  for (int j = 0; j < g.n; ++j) {
    const vdit::Cube c = vdit::cube_at(g, j);
    if (vdit::cube_len_of_flags(g, c.flags) != c.len) return 1;
    std::printf("%d", c.len);
    for (int s = 0; s < c.len; ++s) std::printf(" %d", vdit::cube_token(g, c, s));
    std::printf("\n");
  }
  return 0;
}
