// Schedule of the column loop's trailing update (plain host C++: the CPU tests
// compile it on its own).
//
// The loop runs one launch per 128-column block b; the trailing update after
// block e is W[:, c1:] -= E_e U[c0:c1, c1:] (GPTQ's lazy batches).  The errors
// of block e, E_e, computed in launch e, must reach every column block j > e
// before the launch that quantizes j.  Block e + 1 receives them from the loop
// workgroups of launch e + 1 (the near update, applied to their own rows
// first).  Every other pair (e, j >= e + 2) belongs to a job of the split-bf16
// GEMM tiles that run beside a block's loop: a job applies the errors of the
// consecutive blocks [e0, e0 + ne) to the column blocks j0 .. j1, that is
// W[:, j] -= E[:, e0:e0+ne] U[e0:e0+ne, j] with K = 128 ne.
//
// Two levels, in groups of UPD_LAZY blocks aligned at multiples of UPD_LAZY:
// the errors of block e reach the column blocks up to the first block of the
// next group in launch e + 1 (K = 128, job slot 1); the column blocks past
// that receive the whole group at once, K = 128 UPD_LAZY, in the launch after
// the group's last block (job slot 0).  W's far columns are thus read and
// written once per group instead of once per block.  Every pair (e, j >= e + 2)
// is covered exactly once, in a launch after e and before j, and the jobs of
// one launch touch disjoint column blocks, none of them block b, so nothing in
// a launch depends on another part of it.
#pragma once

#include <stdint.h>

namespace gptq {

struct UpdateJob {
  int64_t e0, ne;  // error blocks [e0, e0 + ne); ne = 0: no job
  int64_t j0, j1;  // column blocks j0 .. j1
};

constexpr int64_t UPD_LAZY = 8;

// The jobs of launch b (1 <= b < nb) of a layer of nb column blocks.
inline void update_jobs(int64_t b, int64_t nb, UpdateJob (&jobs)[2]) {
  jobs[0] = jobs[1] = UpdateJob{0, 0, 0, -1};
  if (b < 1 || b >= nb) return;
  if (b % UPD_LAZY == 0 && b + 1 < nb) jobs[0] = UpdateJob{b - UPD_LAZY, UPD_LAZY, b + 1, nb - 1};
  const int64_t e = b - 1, gend = (e / UPD_LAZY + 1) * UPD_LAZY;  // first block of the next group
  const int64_t j1 = gend < nb - 1 ? gend : nb - 1;
  if (e + 2 <= j1) jobs[1] = UpdateJob{e, 1, e + 2, j1};
}

}  // namespace gptq
