// The large-batch GEMM's 256 x 128 workgroup shape (4 waves x 4 row tiles of
// 16, 2 workgroups per CU; int8 weights, n_out a multiple of 256 but not of
// 512).  The kernel is the one in gemm_prefill.hip; this translation unit is
// always built under the default instruction scheduler: the iterative ILP
// strategy, which gemm_prefill.hip can be built with (WQ_PREFILL_SCHED),
// spills this shape's registers (76-98 VGPRs).
#define WQ_PREFILL_KERNEL_ONLY
#include "gemm_prefill.hip"

namespace wq {

template <int WBITS, bool BF16, int STAGE>
void launch_prefill_n256(const GemmArgs& g, int ksplit, hipStream_t s) {
    launch_prefill_cfg<WBITS, BF16, STAGE, 4, 4, 128, 2>(g, ksplit, s);
}

template void launch_prefill_n256<8, true, STAGE_GATE_UP>(const GemmArgs&, int, hipStream_t);
template void launch_prefill_n256<8, true, STAGE_DOWN>(const GemmArgs&, int, hipStream_t);
template void launch_prefill_n256<8, true, STAGE_RAW>(const GemmArgs&, int, hipStream_t);
template void launch_prefill_n256<8, false, STAGE_GATE_UP>(const GemmArgs&, int, hipStream_t);
template void launch_prefill_n256<8, false, STAGE_DOWN>(const GemmArgs&, int, hipStream_t);
template void launch_prefill_n256<8, false, STAGE_RAW>(const GemmArgs&, int, hipStream_t);

}  // namespace wq
