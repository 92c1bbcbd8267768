// Per-prompt document ranking (BlockRank summary, "Efficient Attention-Based Inference" step 3:
// argmax / arg-top-K of the scores; blog, direct output: a sorted list).
//
// One workgroup per prompt.  The prompt's scores sit in LDS; document k's position in the
// descending order is the number of documents that beat it (a larger score, or an equal score
// and a lower index), so order[position] = k.  This is a stable descending sort by counting:
// O(N^2 / 256) comparisons per thread, exact and deterministic, a few microseconds for the
// N <= 1000 lists re-rankers see.  NaN scores are treated as -infinity.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace br {

struct SortArgs {
  int32_t base[kSortPromptsPerLaunch + 1];  // score index of each prompt's first document
};

__global__ __launch_bounds__(256) void sort_docs_kernel(const float* __restrict__ scores,
                                                        int32_t* __restrict__ order, SortArgs args) {
  __shared__ float s[kSortMaxDocs];
  const int b = blockIdx.x;
  const int base = args.base[b], N = args.base[b + 1] - base;
  for (int k = threadIdx.x; k < N; k += blockDim.x) {
    const float v = scores[base + k];
    s[k] = isnan(v) ? -INFINITY : v;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < N; k += blockDim.x) {
    const float sk = s[k];
    int pos = 0;
    for (int j = 0; j < N; ++j) {
      const float sj = s[j];
      pos += (sj > sk) | ((sj == sk) & (j < k));
    }
    order[base + pos] = k;
  }
}

hipError_t launch_sort_docs(const float* scores, const int32_t* prompt_base, int num_prompts, int32_t* order,
                            hipStream_t stream) {
  for (int p0 = 0; p0 < num_prompts; p0 += kSortPromptsPerLaunch) {
    const int np = num_prompts - p0 < kSortPromptsPerLaunch ? num_prompts - p0 : kSortPromptsPerLaunch;
    SortArgs args;
    for (int b = 0; b <= np; ++b) args.base[b] = prompt_base[p0 + b];
    sort_docs_kernel<<<dim3(unsigned(np)), 256, 0, stream>>>(scores, order, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace br
