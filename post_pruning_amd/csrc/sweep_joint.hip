// In-block sweep with vector-level removal of 16-column ranges (sg_prune_layer_vector).
#include "sweep.h"

namespace sg {

namespace {

template <int MODE, int MGS>
sg_status go(const SweepArgs& a) {
  const void* fn = reinterpret_cast<const void*>(sweep_kernel<MODE, MGS, false, true>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(SweepLds)) != hipSuccess)
    return set_error(SG_ERR_HIP, "hipFuncSetAttribute(sweep_kernel) failed");
  hipLaunchKernelGGL((sweep_kernel<MODE, MGS, false, true>), a.grid, dim3(256), sizeof(SweepLds), a.stream,
                     a.W, a.mask_out, a.Err, a.mask_in, a.st, a.cand, a.parity, a.segs, a.n, a.i1, a.w,
                     a.nkeep, a.mgroup, a.codes_out, a.qscale, a.qzero, a.qlevels);
  return check_launch("prune sweep");
}

}  // namespace

sg_status launch_sweep_joint(const SweepArgs& a) {
  if (a.rpl != 4) return set_error(SG_ERR_UNSUPPORTED, "this sweep takes four rows per lane");
  switch (a.mode) {
    case MODE_THRESH: return go<MODE_THRESH, 0>(a);
    case MODE_FORCED: return go<MODE_FORCED, 0>(a);
    case MODE_ROW: return go<MODE_ROW, 0>(a);
    default:
      switch (a.mgs) {
        case 1: return go<MODE_NM, 1>(a);
        case 2: return go<MODE_NM, 2>(a);
        case 4: return go<MODE_NM, 4>(a);
        case 8: return go<MODE_NM, 8>(a);
        case 16: return go<MODE_NM, 16>(a);
        default: return go<MODE_NM, 0>(a);
      }
  }
}

}  // namespace sg
