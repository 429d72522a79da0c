// In-block sweep with vector-level removal of 16-column ranges (sg_prune_layer_vector).
#include "sweep.h"

namespace sg {

namespace {

template <int MODE, int MGS, int RPL>
sg_status go(const SweepArgs& a) {
  const void* fn = reinterpret_cast<const void*>(sweep_kernel<MODE, MGS, false, true, RPL>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(SweepLds)) != hipSuccess)
    return set_error(SG_ERR_HIP, "hipFuncSetAttribute(sweep_kernel) failed");
  hipLaunchKernelGGL((sweep_kernel<MODE, MGS, false, true, RPL>), a.grid, dim3(256), sizeof(SweepLds), a.stream,
                     a.W, a.mask_out, a.Err, a.mask_in, a.st, a.cand, a.parity, a.segs, a.n, a.i1, a.w,
                     a.nkeep, a.mgroup, a.codes_out, a.qscale, a.qzero, a.qlevels);
  return check_launch("prune sweep");
}

template <int RPL>
sg_status dispatch(const SweepArgs& a) {
  switch (a.mode) {
    case MODE_THRESH: return go<MODE_THRESH, 0, RPL>(a);
    case MODE_FORCED: return go<MODE_FORCED, 0, RPL>(a);
    case MODE_ROW: return go<MODE_ROW, 0, RPL>(a);
    default:
      switch (a.mgs) {
        case 1: return go<MODE_NM, 1, RPL>(a);
        case 2: return go<MODE_NM, 2, RPL>(a);
        case 4: return go<MODE_NM, 4, RPL>(a);
        case 8: return go<MODE_NM, 8, RPL>(a);
        case 16: return go<MODE_NM, 16, RPL>(a);
        default: return go<MODE_NM, 0, RPL>(a);
      }
  }
}

}  // namespace

sg_status launch_sweep_joint(const SweepArgs& a) {
  return a.rpl == 2 ? dispatch<2>(a) : dispatch<4>(a);
}

}  // namespace sg
