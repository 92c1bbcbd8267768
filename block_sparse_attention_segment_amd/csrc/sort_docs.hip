// Per-prompt document ranking (BlockRank summary, "Efficient Attention-Based Inference" step 3:
// argmax / arg-top-K of the scores; blog, direct output: a sorted list).
//
// Each workgroup ranks 64 of one prompt's documents: document k's position in the descending
// order is the number of documents that beat it (a larger score, or an equal score and a lower
// index), so order[position] = k.  This is a stable descending sort by counting, exact and
// deterministic; four threads share each document's N comparisons, and the prompt's scores pass
// through LDS in chunks of kSortChunk, so N is bounded only by the validation limit.
// NaN scores are treated as -infinity.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace br {

struct SortArgs {
  int32_t base[kSortPromptsPerLaunch + 1];  // score index of each prompt's first document
};

constexpr int kSortDocsPerBlock = 64;   // documents ranked per workgroup
constexpr int kSortLanesPerDoc = 4;     // threads sharing one document's comparisons
constexpr int kSortChunk = 8192;        // scores staged in LDS per pass

__device__ __forceinline__ float sort_key(float v) { return isnan(v) ? -INFINITY : v; }

// grid.x = prompt, grid.y = block of 64 documents of that prompt.
__global__ __launch_bounds__(256) void sort_docs_kernel(const float* __restrict__ scores,
                                                        int32_t* __restrict__ order, SortArgs args) {
  __shared__ float s[kSortChunk];
  const int b = blockIdx.x;
  const int base = args.base[b], N = args.base[b + 1] - base;
  const int k0 = blockIdx.y * kSortDocsPerBlock;
  if (k0 >= N) return;  // uniform per workgroup
  const int k = k0 + threadIdx.x / kSortLanesPerDoc, part = threadIdx.x % kSortLanesPerDoc;
  const float sk = k < N ? sort_key(scores[base + k]) : 0.f;
  int pos = 0;
  for (int c0 = 0; c0 < N; c0 += kSortChunk) {
    const int cn = min(kSortChunk, N - c0);
    __syncthreads();  // every thread is done with the previous chunk
    for (int i = threadIdx.x; i < cn; i += blockDim.x) s[i] = sort_key(scores[base + c0 + i]);
    __syncthreads();
    if (k < N) {
      const int kl = k - c0;  // the document's index relative to the chunk
      // Unrolled so that several LDS reads are in flight: the loop is otherwise bound by their
      // latency.  The counts are integers, so the order of the additions does not matter.
#pragma unroll 8
      for (int j = part; j < cn; j += kSortLanesPerDoc) {
        const float sj = s[j];
        pos += (sj > sk) | ((sj == sk) & (j < kl));
      }
    }
  }
  // the 4 lanes of a document are adjacent within one wave
  pos += __shfl_xor(pos, 1);
  pos += __shfl_xor(pos, 2);
  if (k < N && part == 0) order[base + pos] = k;
}

hipError_t launch_sort_docs(const float* scores, const int32_t* prompt_base, int num_prompts, int32_t* order,
                            hipStream_t stream) {
  for (int p0 = 0; p0 < num_prompts; p0 += kSortPromptsPerLaunch) {
    const int np = num_prompts - p0 < kSortPromptsPerLaunch ? num_prompts - p0 : kSortPromptsPerLaunch;
    SortArgs args;
    int max_n = 1;
    for (int b = 0; b <= np; ++b) args.base[b] = prompt_base[p0 + b];
    for (int b = 0; b < np; ++b) max_n = args.base[b + 1] - args.base[b] > max_n ? args.base[b + 1] - args.base[b] : max_n;
    const dim3 grid(unsigned(np), unsigned((max_n + kSortDocsPerBlock - 1) / kSortDocsPerBlock));
    sort_docs_kernel<<<grid, 256, 0, stream>>>(scores, order, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace br
