// Stage 2: per-row top-k block selection.
//
// Cacheon "Kernel ABI", "Attention block slots": attention.decode takes the
// selected nonnegative block ids with -1 meaning none, and
// attention.msa_prefill_block_score leaves unused cells at -1; "Correctness is
// target-owned": selections are graded as sets, so the order within a row is
// free and this library writes ascending block ids.
//
// One wave per score row (select_unit.h holds the selection itself).
#include "device_util.h"
#include "msa_internal.h"
#include "select_unit.h"

namespace msa {

namespace {

template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(TopkParams p) {
    __shared__ __attribute__((aligned(16))) int hist[4][256];
    const int wave = threadIdx.x >> 6;
    const int64_t n = (int64_t)blockIdx.x * 4 + wave;
    if (n >= p.N) return;
    select_row<KPL>(p, n, hist[wave]);
}

template <int KPL>
hipError_t launch(const TopkParams &p, hipStream_t s) {
    const int grid = (p.N + 3) / 4;
    hipLaunchKernelGGL((topk_kernel<KPL>), dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkParams &p, hipStream_t s) {
    if (p.N == 0) return hipSuccess;
    if (p.MB <= 64) return launch<1>(p, s);
    if (p.MB <= 128) return launch<2>(p, s);
    if (p.MB <= 256) return launch<4>(p, s);
    if (p.MB <= 512) return launch<8>(p, s);
    if (p.MB <= 1024) return launch<16>(p, s);
    if (p.MB <= 2048) return launch<32>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace msa
