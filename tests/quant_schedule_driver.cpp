// Prints the trailing-update jobs of quant_schedule.h for tests/test_quant_schedule.py:
// one line per job, "nb b e0 ne j0 j1", for nb = 1 .. argv[1] and every launch
// b = -1 .. nb (launches outside 1 .. nb - 1 must carry no job).
#include <stdio.h>
#include <stdlib.h>

#include "quant_schedule.h"

int main(int argc, char** argv) {
  const long max_nb = argc > 1 ? atol(argv[1]) : 64;
  for (long nb = 1; nb <= max_nb; ++nb)
    for (long b = -1; b <= nb; ++b) {
      gptq::UpdateJob jobs[2];
      gptq::update_jobs(b, nb, jobs);
      for (int k = 0; k < 2; ++k)
        if (jobs[k].ne > 0)
          printf("%ld %ld %lld %lld %lld %lld\n", nb, b, (long long)jobs[k].e0, (long long)jobs[k].ne,
                 (long long)jobs[k].j0, (long long)jobs[k].j1);
    }
  return 0;
}
