// Prints the uint32 stream of rocRAND's Philox-4x32-10 engine (the
// header-only engine of rocrand_kernel.h, compiled here for the host) for a
// seed, a subsequence and an offset: one decimal word per line.  Used by the
// CPU test that pins the oracle's Philox-4x32-10 to an independent
// implementation of the generator.
//
// Usage: rocrand_philox SEED SUBSEQUENCE OFFSET COUNT
#include <rocrand/rocrand_kernel.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) {
    std::fprintf(stderr, "usage: %s SEED SUBSEQUENCE OFFSET COUNT\n", argv[0]);
    return 2;
  }
  const unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
  const unsigned long long sub = std::strtoull(argv[2], nullptr, 0);
  const unsigned long long off = std::strtoull(argv[3], nullptr, 0);
  const long count = std::strtol(argv[4], nullptr, 0);
  rocrand_state_philox4x32_10 state;
  rocrand_init(seed, sub, off, &state);
  for (long i = 0; i < count; ++i) std::printf("%u\n", rocrand(&state));
  return 0;
}
