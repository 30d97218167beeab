// The decode step's top-k selection and its selection-independent attention in
// one launch.
//
// QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制:
// the HCA entries and the sliding window do not depend on which compressed blocks
// the indexer picks.  The selection needs one workgroup per query row for several
// microseconds, so the rest of the chip attends those keys meanwhile: workgroups
// [0, n_sel) of the launch select (as select_kernel), the others attend a split of
// the key range after the CSA picks (as attn_bf16_kernel).  One launch on one
// stream: no cross-queue synchronisation.

#include "attn_impl.hpp"
#include "select_impl.hpp"

namespace v4a {

template <int D>
union StepSmem {
  AttnSmem<D, D == 512> attn;   // rows of 512 are shared entries
  SelShared sel;
};

template <int D, int KP, bool QP, bool F8>
__global__ __launch_bounds__(kSelThreads) void select_attn_kernel(SelectP sp, AttnP ap, int n_sel) {
  static_assert(kSelThreads == 8 * 64, "the attention workgroups run 8 waves");
  __shared__ __align__(16) StepSmem<D> sm;
  const int blk = blockIdx.x;
  if (blk < n_sel) {
    select_row(sp, blk, sm.sel);
    return;
  }
  const int a = blk - n_sel;
  const int xw = ap.splits * ap.head_groups;   // (split, head group) workgroups per row
  attn_block<8, 1, D, KP, QP, D == 512, F8>(ap, a % xw, a / xw, sm.attn, sm.attn.idx);
}

template <int D, int KP>
static void launch_sa(const SelectP& sp, int n_sel, const AttnP& ap, dim3 g, hipStream_t s, int tid) {
  const dim3 blk(kSelThreads);
  constexpr bool CAN_F8 = D <= 128 || D == 512;   // (rows of 512 are shared entries)
  if (CAN_F8 && ap.f8) {
    if (ap.rope_out) V4A_LAUNCH(tid, (select_attn_kernel<D, KP, true, CAN_F8>), g, blk, 0, s, sp, ap, n_sel);
    else V4A_LAUNCH(tid, (select_attn_kernel<D, KP, false, CAN_F8>), g, blk, 0, s, sp, ap, n_sel);
  } else {
    if (ap.rope_out) V4A_LAUNCH(tid, (select_attn_kernel<D, KP, true, false>), g, blk, 0, s, sp, ap, n_sel);
    else V4A_LAUNCH(tid, (select_attn_kernel<D, KP, false, false>), g, blk, 0, s, sp, ap, n_sel);
  }
}

hipError_t launch_select_attn(const SelectP& sp, int n_sel, const AttnP& ap, int n_rows, hipStream_t s, int tid) {
  const int64_t n = (int64_t)n_sel + (int64_t)ap.splits * ap.head_groups * n_rows;
  const int ntile = ap.heads / 16 / max(ap.head_groups, 1);   // head tiles per workgroup
  if (n > INT32_MAX || ap.splits < 1 || ap.heads < 16 || ap.heads > 128 || ap.heads % 16 != 0 ||
      (ap.dim != 64 && ap.dim != 128 && !(ap.dim == 512 && ap.skv)) || ap.head_groups < 1 ||
      ap.heads % (16 * ap.head_groups) != 0)
    return hipErrorInvalidValue;
  const dim3 g((unsigned)n);
  if (ap.dim == 512) {
    // shared rows of 512: a wave pair per head tile, head groups of kWideTiles tiles
    if (ntile > kWideTiles) return hipErrorInvalidValue;
    launch_sa<512, 1>(sp, n_sel, ap, g, s, tid);
  } else if (ntile <= 4) {
    // up to 4 head tiles, two waves per head tile take half of every chunk's keys each
    if (ap.dim == 64) launch_sa<64, 2>(sp, n_sel, ap, g, s, tid);
    else launch_sa<128, 2>(sp, n_sel, ap, g, s, tid);
  } else {
    if (ap.dim == 64) launch_sa<64, 1>(sp, n_sel, ap, g, s, tid);
    else launch_sa<128, 1>(sp, n_sel, ap, g, s, tid);
  }
  return hipGetLastError();
}

}  // namespace v4a
