// The decode step's top-k selection and its selection-independent attention in
// one launch.
//
// QbitAI article "DeepSeek V4报告太详尽了！484天换代之路全公开", section 混合注意力机制:
// the HCA entries and the sliding window do not depend on which compressed blocks
// the indexer picks.  The selection needs one workgroup per query row for several
// microseconds, so the rest of the chip attends those keys meanwhile: workgroups
// [0, n_sel) of the launch select (as select_kernel), the others attend a split of
// the key range after the CSA picks (as attn_bf16_kernel).  One
// launch on one stream: no cross-queue synchronisation.
#include "attn_impl.hpp"
#include "select_impl.hpp"

namespace v4a {

template <int D>
union StepSmem {
  AttnSmem<D> attn;
  SelShared sel;
};

template <int D, int KP>
__global__ __launch_bounds__(kSelThreads) void select_attn_kernel(SelectP sp, AttnP ap, int n_sel) {
  static_assert(kSelThreads == 8 * 64, "the attention workgroups run 8 waves");
  __shared__ __align__(16) StepSmem<D> sm;
  const int blk = blockIdx.x;
  if (blk < n_sel) {
    select_row(sp, blk, sm.sel);
    return;
  }
  const int a = blk - n_sel;
  attn_block<8, 1, D, KP>(ap, a % ap.splits, a / ap.splits, sm.attn);
}

hipError_t launch_select_attn(const SelectP& sp, int n_sel, const AttnP& ap, int n_rows, hipStream_t s,
                              int tid) {
  const int64_t n = (int64_t)n_sel + (int64_t)ap.splits * n_rows;
  if (n > INT32_MAX || ap.splits < 1 || ap.heads < 16 || ap.heads > 128 || ap.heads % 16 != 0)
    return hipErrorInvalidValue;
  // up to 64 heads, two waves per head tile take half of every chunk's keys each
  const dim3 g((unsigned)n), blk(kSelThreads);
  if (ap.heads <= 64) {
    if (ap.dim == 64) V4A_LAUNCH(tid, (select_attn_kernel<64, 2>), g, blk, 0, s, sp, ap, n_sel);
    else V4A_LAUNCH(tid, (select_attn_kernel<128, 2>), g, blk, 0, s, sp, ap, n_sel);
  } else {
    if (ap.dim == 64) V4A_LAUNCH(tid, (select_attn_kernel<64, 1>), g, blk, 0, s, sp, ap, n_sel);
    else V4A_LAUNCH(tid, (select_attn_kernel<128, 1>), g, blk, 0, s, sp, ap, n_sel);
  }
  return hipGetLastError();
}

}  // namespace v4a
