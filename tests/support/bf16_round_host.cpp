// Host build of the library's float/double -> bf16 conversions (f2bf, d2bf in
// msa_internal.h) for the CPU rounding tests: reads a mode byte ('d' doubles
// or 'f' floats) and the values from a file, writes one uint16 per value.
#include <cstdio>
#include <vector>

#include "msa_internal.h"

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  FILE* in = std::fopen(argv[1], "rb");
  if (!in) return 3;
  char mode = 0;
  if (std::fread(&mode, 1, 1, in) != 1) return 4;
  std::vector<uint16_t> out;
  if (mode == 'd') {
    double x;
    while (std::fread(&x, sizeof x, 1, in) == 1) out.push_back(msa::d2bf(x));
  } else if (mode == 'f') {
    float x;
    while (std::fread(&x, sizeof x, 1, in) == 1) out.push_back(msa::f2bf(x));
  } else {
    return 5;
  }
  std::fclose(in);
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) return 6;
  std::fwrite(out.data(), sizeof(uint16_t), out.size(), o);
  std::fclose(o);
  return 0;
}
