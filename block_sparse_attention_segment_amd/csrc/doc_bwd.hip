// Backward of the attention-mass readout and the InfoNCE auxiliary loss on gfx950 (BlockRank
// summary, section 3.4: L_aux = -log(exp(s_gold / tau) / sum_k exp(s_k / tau)), tau = 0.05,
// whose gradient flows back through the readout's attention; blog, attention supervision).
//
//   infonce_kernel    per prompt: loss and g_k = dL/ds_k = (softmax(s / tau)_k - [k = gold]) / tau.
//   doc_center_kernel per (prompt, signal row r): c_r = sum_k mass_rk g_k, with mass_rk the row's
//                     readout weight on document k (from the forward's (m_k, e_k) and (M, 1/Z)).
//   doc_bwd_kernel    one wave per (document group, KV head): streams the group's keys once,
//                     32 at a time inside one document.  With alpha = softmax over the prompt's
//                     document tokens of z = scale Q_S K^T and dz = alpha (g_k(j) - c_r) / Hq:
//                       dQ_S^T += K^T dz^T   (z^T with keys on M, K^T read transposed from LDS)
//                       dK^T    = Q_S^T dz   (z with signal rows on M, Q_S^T read transposed)
//                     Both orientations of z come from the same register fragments.  dK rows of
//                     the keys are written (or added) directly: each key belongs to one group.
//   doc_bwd_reduce_kernel  sums the per-group dQ_S partials of a prompt in a fixed order.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace br {

__global__ __launch_bounds__(256) void infonce_kernel(const float* __restrict__ scores,
                                                      const int32_t* __restrict__ prompt_base,
                                                      const int32_t* __restrict__ gold, float inv_tau,
                                                      float* __restrict__ loss, float* __restrict__ dscores) {
  __shared__ float red[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int k0 = prompt_base[b], N = prompt_base[b + 1] - k0;
  float m = -INFINITY;
  for (int k = tid; k < N; k += 256) m = fmaxf(m, scores[k0 + k] * inv_tau);
  red[tid] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float z = 0.f;
  for (int k = tid; k < N; k += 256) z += expf(scores[k0 + k] * inv_tau - M);
  red[tid] = z;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float lse = M + logf(red[0]);
  const int gd = gold[b];
  for (int k = tid; k < N; k += 256) {
    const float p = expf(scores[k0 + k] * inv_tau - lse);
    dscores[k0 + k] = (p - (k == gd ? 1.f : 0.f)) * inv_tau;
  }
  if (tid == 0) loss[b] = lse - scores[k0 + gd] * inv_tau;
}

// c[b * RT + r] = (1/Z_r) sum_k e_k,r 2^(m_k,r - M_r) g_k over prompt b's documents.  A workgroup
// covers 4 rows x 64 document lanes (the rowstat kernel's layout); the 64 lane sums of a row are
// added in a fixed order.
constexpr int kCenterRows = 4;
constexpr int kCenterLanes = 64;
__global__ __launch_bounds__(256) void doc_center_kernel(const float2* __restrict__ ml,
                                                         const float2* __restrict__ rowstat,
                                                         const int32_t* __restrict__ prompt_base,
                                                         const float* __restrict__ dscores, float* __restrict__ center,
                                                         int RT, int row_groups) {
  __shared__ float red[kCenterRows][kCenterLanes];
  const int b = blockIdx.x / row_groups, rg = blockIdx.x % row_groups;
  const int rl = threadIdx.x % kCenterRows, kl = threadIdx.x / kCenterRows;
  const int r = rg * kCenterRows + rl;
  float c = 0.f;
  if (r < RT) {
    const float M = rowstat[int64_t(b) * RT + r].x;
    for (int k = prompt_base[b] + kl; k < prompt_base[b + 1]; k += kCenterLanes) {
      const float2 v = ml[int64_t(k) * RT + r];
      c = fmaf(v.y * fast_exp2(v.x - M), dscores[k], c);
    }
  }
  red[rl][kl] = c;
  __syncthreads();
  if (kl == 0 && r < RT) {
    float t = 0.f;
    for (int j = 0; j < kCenterLanes; ++j) t += red[rl][j];
    center[int64_t(b) * RT + r] = t * rowstat[int64_t(b) * RT + r].y;
  }
}

template <int D, int RB>
__global__ __launch_bounds__(64) void doc_bwd_kernel(const uint16_t* __restrict__ Q_S, const uint16_t* __restrict__ K,
                                                     const ScoreItem* __restrict__ items, const int32_t* __restrict__ dof,
                                                     const float2* __restrict__ rowstat,
                                                     const float* __restrict__ center, const float* __restrict__ dscores,
                                                     float* __restrict__ dK, float* __restrict__ part, int Hq, int Hkv,
                                                     int n_signal, float scale, float scale_log2, int accumulate) {
  constexpr int DSTEPS = D / 16, DBLK = D / 32, KCH = D / 8;
  constexpr int VROW = D == 128 ? 160 : 96;  // row reads and transposing reads (as V in the forward)
  constexpr int R = RB * 32;                 // signal rows handled (padded)
  constexpr int RBK = 2 * D;             // bytes per K row in LDS (unpadded, 16-byte units swizzled)
  constexpr int UPR = D / 8, KPI = 1024 / RBK, NDMA = 32 / KPI;  // direct-to-LDS: rows per instruction
  __shared__ __align__(1024) uint8_t sk[32 * RBK];
  __shared__ __align__(16) uint16_t sq[R * VROW];
  __shared__ float sM[R], sZ[R], sC[R];

  const int g = blockIdx.x % Hkv;
  const int item = blockIdx.x / Hkv;
  const ScoreItem it = items[item];
  const int lane = threadIdx.x, n = lane & 31, half = lane >> 5;
  const int G = Hq / Hkv, rows = n_signal * G, RT = n_signal * Hq;
  const int64_t kv_stride = int64_t(Hkv) * D;
  const float inv_hq = 1.f / float(Hq);

  // Signal rows of this KV group, row rho = (signal token rho / G, head g G + rho % G), and their
  // readout statistics (M, 1/Z) and centering term c; padding rows get 1/Z = 0, so alpha = 0.
  for (int u = lane; u < R * KCH; u += 64) {
    const int rho = u / KCH, c = u % KCH;
    u32x4_t v = {0, 0, 0, 0};
    if (rho < rows)
      v = load16(Q_S + ((int64_t(it.prompt) * n_signal + rho / G) * Hq + g * G + rho % G) * D + 8 * c);
    *reinterpret_cast<u32x4_t*>(&sq[rho * VROW + 8 * c]) = v;
  }
  for (int rho = lane; rho < R; rho += 64) {
    float m = 0.f, z = 0.f, c = 0.f;
    if (rho < rows) {
      const int64_t ri = int64_t(it.prompt) * RT + (rho / G) * Hq + g * G + rho % G;
      const float2 st = rowstat[ri];
      m = st.x;
      z = st.y;
      c = center[ri];
    }
    sM[rho] = m;
    sZ[rho] = z;
    sC[rho] = c;
  }
  __syncthreads();
  u32x4_t qf[RB][DSTEPS];
  float mN[RB], zN[RB], cN[RB];  // this lane's row (N index) of each row block
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) qf[rb][s] = load16(&sq[(32 * rb + n) * VROW + 16 * s + 8 * half]);
    mN[rb] = sM[32 * rb + n];
    zN[rb] = sZ[32 * rb + n];
    cN[rb] = sC[32 * rb + n];
  }
  // Transposing-read lane pattern (the forward's V^T reads): 16-lane group s = lane % 16,
  // head-dim half (lane / 16) % 2, row half `half`.
  const int vs = lane & 15, vdh = (lane >> 4) & 1;
  const int t_lane = (4 * half + (vs >> 2)) * VROW + 16 * vdh + 4 * (vs & 3);
  // The K tile: row r at RBK r bytes, 16-byte unit c at c ^ swz(r), which keeps both its row reads
  // (16 keys at one unit) and its transposing reads (4 keys x 2 unit pairs per half-wave, keys + 8
  // with the swizzle ^ 2) free of bank conflicts; it repeats every 16 rows.
  auto swz = [](int r) { return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3); };
  uint32_t kro[DSTEPS];  // row reads: key n, unit 2 s + half
#pragma unroll
  for (int st = 0; st < DSTEPS; ++st) kro[st] = uint32_t(n * RBK + 16 * ((2 * st + half) ^ swz(n)));
  const int tr_r = 4 * half + (vs >> 2);
  uint32_t ktl[DBLK], kth[DBLK];  // transposing reads: keys tr_r (+ 8), head-dim element 32 b + 16 vdh + 4 (vs % 4)
#pragma unroll
  for (int b = 0; b < DBLK; ++b) {
    const int unit = 4 * b + 2 * vdh + ((vs & 3) >> 1);
    ktl[b] = uint32_t(tr_r * RBK + 16 * (unit ^ swz(tr_r)) + 8 * (vs & 1));
    kth[b] = uint32_t((tr_r + 8) * RBK + 16 * (unit ^ swz(tr_r + 8)) + 8 * (vs & 1));
  }
  // Direct-to-LDS loads of a 32-key block: instruction i fills LDS bytes [1 KB i, 1 KB (i + 1)):
  // lane l unit l % UPR of key row KPI i + l / UPR, from source unit (l % UPR) ^ swz(row).  Keys
  // past the document's end load as zeros.
  const uint32_t sk_lds = lds_addr_of(sk);
  auto issue_k = [&](int t0, int nk) {
    t0 = __builtin_amdgcn_readfirstlane(t0);
    nk = __builtin_amdgcn_readfirstlane(nk);
    const rsrc_t r = make_rsrc(K + int64_t(t0) * kv_stride + g * D, nk * int(kv_stride) * 2);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int row = KPI * i + lane / UPR, c = (lane % UPR) ^ swz(row);
      buf_load16_lds(r, sk_lds + 1024 * i, uint32_t(row * int(kv_stride) * 2 + 16 * c));
    }
  };

  f32x16_t aq[RB][DBLK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int b = 0; b < DBLK; ++b) aq[rb][b] = f32x16_t{};

  // Blocks of 32 keys inside each document of the group, in order.  Block i + 1's keys are loaded
  // into the (single) K tile as soon as block i's last read of it is done, so that load overlaps
  // block i's dK read-modify-write and stores.
  if (it.d0 < it.d1) issue_k(dof[it.d0], min(32, dof[it.d0 + 1] - dof[it.d0]));
  bool first = true;
  for (int d = it.d0; d < it.d1; ++d) {
    const int a = dof[d], e = dof[d + 1];
    const float gk = dscores[it.score_base + (d - it.d0)];
    for (int t0 = a; t0 < e; t0 += 32) {
      const int nk = min(32, e - t0);
      // This block's keys have landed: all that was issued after them is the previous block's
      // dK stores (its dK loads were consumed before the stores).
      if (first) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else if constexpr (D == 128) {
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      }
      first = false;
      u32x4_t kf[DSTEPS];
#pragma unroll
      for (int s = 0; s < DSTEPS; ++s) kf[s] = load16(sk + kro[s]);
      f32x16_t ak[DBLK];
#pragma unroll
      for (int b = 0; b < DBLK; ++b) ak[b] = f32x16_t{};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // z^T: keys on M (register r: key t0 + 8 (r / 4) + 4 half + r % 4), this lane's row on N.
        f32x16_t zt = f32x16_t{}, z = f32x16_t{};
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) {
          zt = mfma32(kf[s], qf[rb][s], zt);
          z = mfma32(qf[rb][s], kf[s], z);
        }
        uint32_t pk[8], pd[8];
        const float wN = (gk - cN[rb]) * inv_hq;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int kk = 8 * (r >> 2) + 4 * half + (r & 3);
          const float a0 = kk < nk ? fast_exp2(fmaf(zt[r], scale_log2, -mN[rb])) * zN[rb] : 0.f;
          const float a1 = kk + 1 < nk ? fast_exp2(fmaf(zt[r + 1], scale_log2, -mN[rb])) * zN[rb] : 0.f;
          pk[r >> 1] = pack_bf16x2(a0 * wN, a1 * wN);
          // z: signal rows on M (register r: row 32 rb + kk), this lane's key on N.
          const int r0 = 32 * rb + kk;
          const float b0 = fast_exp2(fmaf(z[r], scale_log2, -sM[r0])) * sZ[r0] * (gk - sC[r0]) * inv_hq;
          const float b1 = fast_exp2(fmaf(z[r + 1], scale_log2, -sM[r0 + 1])) * sZ[r0 + 1] * (gk - sC[r0 + 1]) * inv_hq;
          pd[r >> 1] = pack_bf16x2(b0, b1);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const u32x4_t bk = {pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]};
          const u32x4_t bq = {pd[4 * m], pd[4 * m + 1], pd[4 * m + 2], pd[4 * m + 3]};
          const uint8_t* kt = sk + 16 * m * RBK;
          const uint16_t* qt = &sq[t_lane + (32 * rb + 16 * m) * VROW];
#pragma unroll
          for (int b = 0; b < DBLK; ++b) {
            const u32x2_t klo = lds_read_tr16(reinterpret_cast<const uint16_t*>(kt + ktl[b]));
            const u32x2_t khi = lds_read_tr16(reinterpret_cast<const uint16_t*>(kt + kth[b]));
            aq[rb][b] = mfma32(u32x4_t{klo[0], klo[1], khi[0], khi[1]}, bk, aq[rb][b]);
            const u32x2_t qlo = lds_read_tr16(qt + 32 * b), qhi = lds_read_tr16(qt + 8 * VROW + 32 * b);
            ak[b] = mfma32(u32x4_t{qlo[0], qlo[1], qhi[0], qhi[1]}, bq, ak[b]);
          }
        }
      }
      // Every read of this block's K tile is done: load the next block's keys into it.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      {
        int nt0 = t0 + 32, nd = d;
        if (nt0 >= e) {
          ++nd;
          nt0 = nd < it.d1 ? dof[nd] : 0;
        }
        if (nd < it.d1) issue_k(nt0, min(32, dof[nd + 1] - nt0));
      }
      // ak[b] register r: head-dim element 32 b + 8 (r / 4) + 4 half + r % 4 of key t0 + n.
      if (n < nk) {
        float* dst = dK + (int64_t(t0 + n) * Hkv + g) * D + 4 * half;
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f32x4_t v = f32x4_t{ak[b][4 * j], ak[b][4 * j + 1], ak[b][4 * j + 2], ak[b][4 * j + 3]} * scale;
            f32x4_t* p = reinterpret_cast<f32x4_t*>(dst + 32 * b + 8 * j);
            if (accumulate) v += *p;
            *p = v;
          }
      }
    }
  }
  // aq[rb][b] register r: head-dim element 32 b + 8 (r / 4) + 4 half + r % 4 of row 32 rb + n.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float* dst = part + ((int64_t(item) * Hkv + g) * RB + rb) * 32 * D + n * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4_t*>(dst + 32 * b + 8 * j) =
            f32x4_t{aq[rb][b][4 * j], aq[rb][b][4 * j + 1], aq[rb][b][4 * j + 2], aq[rb][b][4 * j + 3]} * scale;
  }
}

// dQ_S[b, i, h, :] = sum over prompt b's items of the group partials.  One workgroup per
// (prompt, KV head, signal row): 8 item slices x (D / 4) element groups; each slice sums every
// 8th item and the slices are added in a fixed order (deterministic).
constexpr int kReduceSlices = 8;
template <int D>
__global__ __launch_bounds__(kReduceSlices * D / 4) void doc_bwd_reduce_kernel(const float* __restrict__ part,
                                                                             const int32_t* __restrict__ prompt_items,
                                                                             float* __restrict__ dQ_S, int Hq, int Hkv,
                                                                             int n_signal, int RB) {
  constexpr int CH = D / 4;
  __shared__ f32x4_t red[kReduceSlices][CH];
  const int R = RB * 32;
  const int rho = blockIdx.x % R;
  const int g = (blockIdx.x / R) % Hkv;
  const int b = blockIdx.x / (R * Hkv);
  const int G = Hq / Hkv;
  if (rho >= n_signal * G) return;  // uniform per workgroup
  const int ch = threadIdx.x % CH, sl = threadIdx.x / CH;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t item_stride = int64_t(Hkv) * RB * 32 * D;
  const float* src = part + (int64_t(g) * RB + rho / 32) * 32 * D + (rho % 32) * D + 4 * ch;
  // Unrolled so that eight loads are in flight; the additions stay in item order.
#pragma unroll 8
  for (int i = prompt_items[b] + sl; i < prompt_items[b + 1]; i += kReduceSlices)
    acc += *reinterpret_cast<const f32x4_t*>(src + int64_t(i) * item_stride);
  red[sl][ch] = acc;
  __syncthreads();
  if (sl == 0) {
    f32x4_t t = red[0][ch];
    for (int j = 1; j < kReduceSlices; ++j) t += red[j][ch];
    *reinterpret_cast<f32x4_t*>(dQ_S + ((int64_t(b) * n_signal + rho / G) * Hq + g * G + rho % G) * D + 4 * ch) = t;
  }
}

hipError_t launch_infonce(const float* scores, const int32_t* prompt_base, const int32_t* gold, float tau,
                          int num_prompts, float* loss, float* dscores, hipStream_t stream) {
  infonce_kernel<<<unsigned(num_prompts), 256, 0, stream>>>(scores, prompt_base, gold, 1.f / tau, loss, dscores);
  return hipGetLastError();
}

template <int D, int RB>
static hipError_t launch_doc_bwd_t(const DocBwdLaunch& a, hipStream_t stream) {
  const int RT = a.n_signal * a.num_q_heads;
  const int row_groups = (RT + kCenterRows - 1) / kCenterRows;
  doc_center_kernel<<<unsigned(a.num_prompts * row_groups), 256, 0, stream>>>(a.ml, a.rowstat, a.prompt_base,
                                                                              a.dscores, a.center, RT, row_groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  doc_bwd_kernel<D, RB><<<unsigned(a.n_items * a.num_kv_heads), 64, 0, stream>>>(
      a.Q_S, a.K, a.items, a.doc_offsets, a.rowstat, a.center, a.dscores, a.dK, a.part, a.num_q_heads, a.num_kv_heads,
      a.n_signal, a.scale, a.scale * kLog2e, a.accumulate);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  doc_bwd_reduce_kernel<D><<<unsigned(a.num_prompts * a.num_kv_heads * RB * 32), kReduceSlices * D / 4, 0, stream>>>(
      a.part, a.prompt_items, a.dQ_S, a.num_q_heads, a.num_kv_heads, a.n_signal, RB);
  return hipGetLastError();
}

hipError_t launch_doc_bwd(const DocBwdLaunch& a, hipStream_t stream) {
  if (a.head_dim == 128) return a.row_blocks == 1 ? launch_doc_bwd_t<128, 1>(a, stream) : launch_doc_bwd_t<128, 2>(a, stream);
  return a.row_blocks == 1 ? launch_doc_bwd_t<64, 1>(a, stream) : launch_doc_bwd_t<64, 2>(a, stream);
}

}  // namespace br
