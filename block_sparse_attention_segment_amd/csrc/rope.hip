// Rotary position embedding with BlockRank's permutation-invariant position ids.
//
// Positions (BlockRank summary, section 3.4 "Permutation-invariant position embeddings"):
// instruction token i sits at i, token j of every document at j + (instruction length), so a
// document's positions do not depend on its place in the list, and the final query starts at a
// fixed offset (8192 there; BlockSearch, section 3.2, restarts every document at 0 and puts the
// query at 300).  The host turns the segment table into runs of consecutive positions; this
// kernel finds a row's run by binary search.
//
// Rotation (RoFormer): pair k of a head vector turns by pos * theta^(-2k/d).  Pairs are either
// the two halves (k, k + d/2) or adjacent entries (2k, 2k + 1).  The angle is formed and reduced
// modulo 2*pi in fp64 (positions reach 10^4 radians and more), then sin/cos and the rotation run
// in fp32 and the result is rounded to bf16.
//
// Work: one thread per (row, group of 8 pairs); it computes its 8 sin/cos pairs once and rotates
// those pairs in every Q head and every K head of the row.  HBM-bound: each element is read and
// written once, 16-byte vector accesses, a row's heads contiguous.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace br {

constexpr double kRopeTwoPi = 6.283185307179586476925286766559;
constexpr double kRopeInvTwoPi = 0.15915494309189533576888376337251;

// cos and sin of pos * inv_freq: the angle is formed and reduced modulo 2*pi in fp64, sin/cos in
// fp32 (shared by the rotation kernel and the cos/sin table of the attention's fused rotation).
__device__ __forceinline__ void rope_cos_sin(double pos, double inv_freq, float* cs, float* sn) {
  const double ang = pos * inv_freq;
  const double turns = rint(ang * kRopeInvTwoPi);
  const float r = float(fma(-turns, kRopeTwoPi, ang));
  sincosf(r, sn, cs);
}

struct RopeArgs {
  const uint16_t* q;
  uint16_t* q_out;
  const uint16_t* k;
  uint16_t* k_out;
  const int32_t* run_start;
  const int32_t* run_pos0;
  const double* inv_freq;
  int64_t rows;
  int n_runs, q_heads, k_heads;
};

// Rotate the 8 pairs of one head: x0 and x1 hold the pairs' first and second entries (split
// layout) or eight interleaved (first, second) entries over two vectors (adjacent layout).
template <bool kAdjacent>
__device__ __forceinline__ void rope_rotate8(u32x4_t& x0, u32x4_t& x1, const float* cs, const float* sn) {
  if constexpr (!kAdjacent) {
    rope_rotate_split8(x0, x1, cs, sn);
  } else {
    rope_rotate_adjacent4(x0, cs, sn);          // pairs 0..3
    rope_rotate_adjacent4(x1, cs + 4, sn + 4);  // pairs 4..7
  }
}

template <int D, bool kAdjacent>
__device__ __forceinline__ void rope_rotate_heads(const uint16_t* src, uint16_t* dst, int heads, int64_t row, int c,
                                             const float* cs, const float* sn) {
  // element offsets of this thread's two 16-byte pieces inside a head vector
  const int o0 = kAdjacent ? 16 * c : 8 * c;
  const int o1 = kAdjacent ? 16 * c + 8 : D / 2 + 8 * c;
  const int64_t base = row * heads * D;
  // Every element is read once and written once: both with the non-temporal hint (whole
  // 128-byte lines: eight threads cover each half of a head vector).
  constexpr int U = 4;
  int h = 0;
  for (; h + U <= heads; h += U) {
    u32x4_t x0[U], x1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      x0[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + base + int64_t(h + u) * D + o0));
      x1[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + base + int64_t(h + u) * D + o1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      rope_rotate8<kAdjacent>(x0[u], x1[u], cs, sn);
      __builtin_nontemporal_store(x0[u], reinterpret_cast<u32x4_t*>(dst + base + int64_t(h + u) * D + o0));
      __builtin_nontemporal_store(x1[u], reinterpret_cast<u32x4_t*>(dst + base + int64_t(h + u) * D + o1));
    }
  }
  for (; h < heads; ++h) {
    u32x4_t x0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + base + int64_t(h) * D + o0));
    u32x4_t x1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + base + int64_t(h) * D + o1));
    rope_rotate8<kAdjacent>(x0, x1, cs, sn);
    __builtin_nontemporal_store(x0, reinterpret_cast<u32x4_t*>(dst + base + int64_t(h) * D + o0));
    __builtin_nontemporal_store(x1, reinterpret_cast<u32x4_t*>(dst + base + int64_t(h) * D + o1));
  }
}

template <int D, bool kAdjacent>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
  constexpr int kGroups = D / 16;          // groups of 8 pairs per head vector
  constexpr int kRowsPerBlock = 256 / kGroups;
  const int c = int(threadIdx.x) % kGroups;
  const int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + int(threadIdx.x) / kGroups;
  if (row >= a.rows) return;
  // run holding this row: the last r with run_start[r] <= row
  int lo = 0, hi = a.n_runs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.run_start[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const double pos = double(a.run_pos0[lo]) + double(row - a.run_start[lo]);
  float cs[8], sn[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rope_cos_sin(pos, a.inv_freq[8 * c + j], &cs[j], &sn[j]);  // 8 consecutive pairs
  if (a.q_heads) rope_rotate_heads<D, kAdjacent>(a.q, a.q_out, a.q_heads, row, c, cs, sn);
  if (a.k_heads) rope_rotate_heads<D, kAdjacent>(a.k, a.k_out, a.k_heads, row, c, cs, sn);
}

namespace {

template <int D, bool kAdjacent>
hipError_t launch(const RopeArgs& a, hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / (D / 16);
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  rope_kernel<D, kAdjacent><<<dim3(unsigned(blocks)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

// Table of cos/sin per distinct position: table row t is position iv_pos0[i] + (t - iv_off[i])
// for the interval i holding row t; entry [t][k] = (cos, sin) of pair k.  One thread per entry.
__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* __restrict__ iv_pos0,
                                                         const int32_t* __restrict__ iv_off, int n_iv, int64_t rows,
                                                         int half, const double* __restrict__ inv_freq,
                                                         float2* __restrict__ table) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= rows * half) return;
  const int64_t t = e / half;
  const int k = int(e % half);
  int lo = 0, hi = n_iv - 1;  // the last interval starting at or before row t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (iv_off[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const double pos = double(iv_pos0[lo]) + double(t - iv_off[lo]);
  float cs, sn;
  rope_cos_sin(pos, inv_freq[k], &cs, &sn);
  table[e] = float2{cs, sn};
}

hipError_t launch_rope_table(const int32_t* iv_pos0, const int32_t* iv_off, int n_iv, int64_t rows, int head_dim,
                             const double* inv_freq, float* table, hipStream_t stream) {
  const int64_t n = rows * (head_dim / 2);
  if (n <= 0) return hipSuccess;
  rope_table_kernel<<<dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream>>>(
      iv_pos0, iv_off, n_iv, rows, head_dim / 2, inv_freq, reinterpret_cast<float2*>(table));
  return hipGetLastError();
}

hipError_t launch_rope(const RopeLaunch& l, hipStream_t stream) {
  if (l.rows <= 0 || (l.q_heads == 0 && l.k_heads == 0)) return hipSuccess;
  RopeArgs a{l.q, l.q_out, l.k, l.k_out, l.run_start, l.run_pos0, l.inv_freq, l.rows, l.n_runs, l.q_heads, l.k_heads};
  if (l.head_dim == 128) return l.adjacent ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return l.adjacent ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace br
