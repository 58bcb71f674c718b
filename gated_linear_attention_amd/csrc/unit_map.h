// Workgroup -> (sequence, query head, kv head, V tile) for the chunk kernels.
//
// The runtime deals the workgroups of a launch to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8), and each XCD has its own L2.  The work is
// grouped by (sequence, kv head): with grouped kv heads the n_rep = H / Hkv
// query heads of one kv head read the same k and v rows, and the V tiles of
// one query head read the same q and k rows.  A group goes to one XCD, its
// n_rep * nvt workgroups adjacent in that XCD's dispatch order, so those
// repeated reads are served by that XCD's L2.  With n_rep == 1 and nvt == 1
// this is plain round-robin over (sequence, head).
#pragma once

#include <hip/hip_runtime.h>

#include "sgla_internal.h"

namespace sgla {

struct UnitMap {
  int32_t rank;   // row of the sequence table (dense: batch row)
  int32_t hd;     // query head
  int32_t hk;     // kv head = hd / n_rep
  int32_t vt;     // V tile
  bool valid;     // false for the padding workgroups of the last XCD round
};

// Inverse of the order described above; the grid has
// unit_grid(num_seqs, Hkv, n_rep, nvt) workgroups.
__device__ __forceinline__ UnitMap map_unit(int32_t bid, int32_t nvt, int32_t Hkv, int32_t n_rep,
                                            int32_t num_seqs) {
  const int32_t xcd = bid % kXcds;
  const int32_t slot = bid / kXcds;
  const int32_t qs = slot / nvt;            // (group, member) slot on this XCD
  const int32_t gs = qs / n_rep;
  const int32_t grp = gs * kXcds + xcd;     // rank * Hkv + hk
  UnitMap u;
  u.vt = slot - qs * nvt;
  u.valid = grp < num_seqs * Hkv;
  u.rank = grp / Hkv;
  u.hk = grp - u.rank * Hkv;
  u.hd = u.hk * n_rep + (qs - gs * n_rep);
  return u;
}

}  // namespace sgla
