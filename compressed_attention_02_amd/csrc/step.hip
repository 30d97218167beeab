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
//
// In the one-launch form, when the whole grid fits the chip at once, the launch
// also attends the picks and merges: the selecting workgroup publishes its row
// (agent-scope release of a row word), the workgroups of the picks wait for it
// before reading idx; the other attention workgroups of a row, done long before
// the selection, wait for each other and combine their partials into one per head;
// then every attention workgroup of the row counts itself done, waits for the
// row's last split and merges a share of the heads.  Waits are bounded in time; a
// wait that gives up leaves NaN in the outputs it owns rather than hang.
#include "attn_impl.hpp"
#include "select_impl.hpp"

namespace v4a {

template <int D>
union StepSmem {
  AttnSmem<D, D == 512> attn;   // rows of 512 are shared entries
  SelShared sel;
};

template <int D, int KP, bool QP, bool F8>
__global__ __launch_bounds__(kSelThreads) void select_attn_kernel(SelectP sp, AttnP ap, AttnP csa, int n_sel,
                                                                  int n_rest) {
  static_assert(kSelThreads == 8 * 64, "the attention workgroups run 8 waves");
  __shared__ __align__(16) StepSmem<D> sm;
  const int blk = blockIdx.x;
  if (blk < n_sel) {
    select_row(sp, blk, sm.sel);
    if (csa.sync) wg_release(csa.sync + kRowWords * blk, true);  // publish the row's picks
    return;
  }
  const int a = blk - n_sel;
  if (a < n_rest) {
    const int xw = ap.splits * ap.head_groups;   // (split, head group) workgroups per row
    attn_block<8, 1, D, KP, true, QP, D == 512, F8>(ap, a % xw, a / xw, sm.attn);
  } else {
    const int c = a - n_rest;
    attn_block<8, 1, D, KP, true, QP, D == 512, F8>(csa, c % csa.splits, c / csa.splits, sm.attn);
  }
}

template <int D, int KP>
static void launch_sa(const SelectP& sp, int n_sel, const AttnP& ap, const AttnP& csa, int nr, dim3 g,
                      hipStream_t s, int tid) {
  const dim3 blk(kSelThreads);
  constexpr bool CAN_F8 = D <= 128;
  if (CAN_F8 && ap.f8) {
    if (ap.rope_out) V4A_LAUNCH(tid, (select_attn_kernel<D, KP, true, CAN_F8>), g, blk, 0, s, sp, ap, csa, n_sel, nr);
    else V4A_LAUNCH(tid, (select_attn_kernel<D, KP, false, CAN_F8>), g, blk, 0, s, sp, ap, csa, n_sel, nr);
  } else {
    if (ap.rope_out) V4A_LAUNCH(tid, (select_attn_kernel<D, KP, true, false>), g, blk, 0, s, sp, ap, csa, n_sel, nr);
    else V4A_LAUNCH(tid, (select_attn_kernel<D, KP, false, false>), g, blk, 0, s, sp, ap, csa, n_sel, nr);
  }
}

int64_t select_attn_grid(int n_sel, const AttnP& ap, const AttnP& csa, int n_rows) {
  return (int64_t)n_sel + ((int64_t)ap.splits * ap.head_groups + (csa.sync ? csa.splits : 0)) * n_rows;
}

hipError_t launch_select_attn(const SelectP& sp, int n_sel, const AttnP& ap, const AttnP& csa, int n_rows,
                              hipStream_t s, int tid) {
  const int64_t n = select_attn_grid(n_sel, ap, csa, n_rows);
  const int64_t n_rest = (int64_t)ap.splits * ap.head_groups * n_rows;
  if (n > INT32_MAX || ap.splits < 1 || ap.heads < 16 || ap.heads > 128 || ap.heads % 16 != 0 ||
      (ap.dim != 64 && ap.dim != 128 && !(ap.dim == 512 && ap.skv && !ap.sync)) ||
      (ap.dim != 512 && ap.head_groups != 1) || ap.head_groups < 1 || (csa.sync && csa.head_groups != 1))
    return hipErrorInvalidValue;
  // the rest pre-merge needs the row words; with the picks attended in the same
  // launch both parts carry them, the picks' part waits for the selection, and
  // every split joins the final merge
  if (ap.premerge && (!ap.sync || ap.splits < 2 || ap.splits > kStepMaxSplits ||
                      ap.merge_lo != ap.split_base + ap.splits - 1))
    return hipErrorInvalidValue;
  if (csa.sync && (csa.splits < 1 || ap.sync != csa.sync || !csa.wait_idx || ap.wait_idx || !ap.final_merge ||
                   !csa.final_merge || ap.splits_total != ap.splits + csa.splits ||
                   csa.splits_total != ap.splits_total || ap.splits_total > kStepMaxSplits ||
                   ap.merge_lo != csa.merge_lo))
    return hipErrorInvalidValue;
  if (!csa.sync && ap.final_merge) return hipErrorInvalidValue;
  // up to 64 heads, two waves per head tile take half of every chunk's keys each
  const dim3 g((unsigned)n);
  const int nr = (int)n_rest;
  if (ap.dim == 512) {
    // shared rows of 512: a wave pair per head tile, head groups of kWideTiles tiles
    if (ap.heads / 16 / ap.head_groups > kWideTiles) return hipErrorInvalidValue;
    launch_sa<512, 1>(sp, n_sel, ap, csa, nr, g, s, tid);
  } else if (ap.heads <= 64) {
    if (ap.dim == 64) launch_sa<64, 2>(sp, n_sel, ap, csa, nr, g, s, tid);
    else launch_sa<128, 2>(sp, n_sel, ap, csa, nr, g, s, tid);
  } else {
    if (ap.dim == 64) launch_sa<64, 1>(sp, n_sel, ap, csa, nr, g, s, tid);
    else launch_sa<128, 1>(sp, n_sel, ap, csa, nr, g, s, tid);
  }
  return hipGetLastError();
}

}  // namespace v4a
