// Prints Philox4x32-10 words from rocRAND's own generator state, run on the
// host.  Used only to pin the CPU oracle's Philox implementation.
// usage: rocrand_philox_ref <seed> <subsequence> <offset> <count>
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_kernel.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  unsigned long long seed = strtoull(argv[1], nullptr, 0);
  unsigned long long sub = strtoull(argv[2], nullptr, 0);
  unsigned long long off = strtoull(argv[3], nullptr, 0);
  long count = strtol(argv[4], nullptr, 0);
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, sub, off, &st);
  for (long i = 0; i < count; i++) printf("%u\n", rocrand(&st));
  return 0;
}
