// Backward of the block-sparse prefill attention on gfx950 (MI355X).
//
// For O = softmax(scale Q K^T + M) V with the BlockRank mask M (BlockRank summary, section 3.4;
// the auxiliary loss there sends its gradient back through this attention), given dO and the
// forward's log-sum-exp L per row:
//   P  = exp(scale Q K^T - L)   on allowed pairs, 0 elsewhere (recomputed, never stored)
//   Dr = rowsum(dO * O)          (= rowsum(P * dP), the softmax Jacobian's row term)
//   dP = dO V^T,  dS = P * (dP - Dr)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// Only allowed (row, key) pairs are visited, through the same host plans as the forward:
//   attn_bwd_dq_kernel   query-major over the forward plan's row tiles (128 (token, head) rows,
//                        4 waves of 32 rows); it also forms Dr (and -lse log2 e) for its rows.
//                        Per 64-key tile, loaded straight into LDS while the previous one is
//                        used: S^T = K Q^T and dP^T = V dO^T (keys on M), dS^T in fp32,
//                        dQ^T += K^T dS^T with dS rounded to bf16 and K^T fragments from
//                        transposing LDS reads (as V^T in the forward).
//   attn_bwd_dkv_kernel  key-major: 64 keys of one KV head per workgroup (4 waves of 16 keys,
//                        16x16x32 products); the rows that read them stream through LDS 64
//                        (token, head) rows at a time by direct-to-LDS loads, the next step's
//                        in flight: S = Q K^T and dP = dO V^T (rows on M), then dV^T += dO^T P
//                        and dK^T += Q^T dS with the row-side operands read transposed from LDS.
// Long row or key ranges are split; their fp32 partials are summed by the merge kernels in a
// fixed order, so results are deterministic.  Outputs are fp32.  Both kernels stage their fp32
// rows through LDS so that every store writes whole rows, and store them with the non-temporal
// hint: nothing reads them again in this pass.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace br {

template <int D, int G>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
                                                          const uint16_t* __restrict__ dO,
                                                          const float* __restrict__ lse, float* __restrict__ dvec,
                                                          float* __restrict__ nlse2,
                                                          float* __restrict__ dQ, const AttnItem* __restrict__ items,
                                                          float* __restrict__ part_dq, int Hq, int Hkv, float scale,
                                                          float scale_log2) {
  constexpr int TM = kRowsPerTile / G;
  constexpr int BN = kKeyTile;
  constexpr int NKB = BN / 32;
  constexpr int RB = 2 * D;           // bytes per K or V row
  constexpr int UPR = D / 8;          // 16-byte units per row
  constexpr int KPI = 1024 / RB;      // key rows per direct-to-LDS wave instruction
  constexpr int NDMA = BN / KPI / 4;  // such instructions per wave per tensor per tile
  constexpr int TB = BN * RB;         // bytes per K or V tile
  constexpr int DSTEPS = D / 16, DBLK = D / 32;
  static_assert(NDMA >= 1 && NDMA * KPI * 4 == BN, "a tile's rows split over four waves");
  static_assert(4 * TB >= kRowsPerTile * 4 * D, "the output rows fit in the tile buffers");
  // LDS: the K and V tiles of two slots (tile i in slot i % 2 while tile i + 1 loads into the
  // other, one barrier per tile); after the last tile, each wave's 32 fp32 output rows.
  __shared__ __align__(1024) uint8_t lds[4 * TB];
  // Swizzles of the 16-byte units of a row: K is read by rows (16 keys at one unit) and by
  // transposing reads (4 keys x 2 unit pairs per half-wave, keys + 8 with the swizzle ^ 2); V by
  // rows only.  Both repeat every 16 rows.
  auto swz_k = [](int r) { return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3); };
  auto swz_v = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };

  const int g = blockIdx.x % Hkv;
  const AttnItem it = items[blockIdx.x / Hkv];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, half = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int rho = w * 32 + n, hh = rho / TM, tt = rho % TM, h = g * G + hh;
  const int row_tok = it.row0 + tt;
  const bool row_ok = row_tok < it.row_limit;
  const int q_stride = Hq * D, kv_stride = Hkv * D;

  // This lane's row: Q and dO fragments (B operands of S^T and dP^T), log2-domain lse, Dr.
  const int rows = min(TM, it.row_limit - it.row0);
  const rsrc_t rq = make_rsrc(Q + (int64_t(it.row0) * Hq + g * G) * D, rows * q_stride * 2);
  const rsrc_t rdo = make_rsrc(dO + (int64_t(it.row0) * Hq + g * G) * D, rows * q_stride * 2);
  const uint32_t q_off = uint32_t((tt * q_stride + hh * D + 8 * half) * 2);
  u32x4_t qf[DSTEPS], df[DSTEPS];
#pragma unroll
  for (int s = 0; s < DSTEPS; ++s) {
    qf[s] = buf_load16(rq, q_off + 32 * s);
    df[s] = buf_load16(rdo, q_off + 32 * s);
  }
  const int64_t rix = int64_t(row_tok) * Hq + h;
  const float l2 = row_ok ? lse[rix] * kLog2e : 0.f;
  // Dr = rowsum(dO * O) for this lane's row: each lane half holds 64 of the row's elements.  The
  // item that owns the row's output (a direct tile, or the split chunk that carries the causal
  // part) also stores it for the key-major kernel that runs next.
  float dr;
  {
    const rsrc_t ro = make_rsrc(O + (int64_t(it.row0) * Hq + g * G) * D, rows * q_stride * 2);
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) {
      const u32x4_t ov = buf_load16(ro, q_off + 32 * s);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = fmaf(__uint_as_float(ov[j] << 16), __uint_as_float(df[s][j] << 16), acc0);
        acc1 = fmaf(__uint_as_float(ov[j] & 0xffff0000u), __uint_as_float(df[s][j] & 0xffff0000u), acc1);
      }
    }
    dr = acc0 + acc1;
    dr += other_half(dr);
    if (row_ok && half == 0 && (it.slot < 0 || it.b_end > it.b_start)) {
      dvec[rix] = dr;
      nlse2[rix] = -l2;  // the key-major kernel's exponent offset
    }
  }

  // Row reads (A operands of S^T and dP^T): key 32 kb + n, unit 2 st + half.
  uint32_t kro[DSTEPS], vro[DSTEPS];
#pragma unroll
  for (int st = 0; st < DSTEPS; ++st) {
    kro[st] = uint32_t(n * RB + 16 * ((2 * st + half) ^ swz_k(n)));
    vro[st] = uint32_t(n * RB + 16 * ((2 * st + half) ^ swz_v(n)));
  }
  // K^T fragments for dQ^T += K^T dS^T (transposing reads, the forward's V^T pattern): in each
  // 16-lane group, lane s points at key 4 half + s / 4 (+ 8 for the upper four) and head-dim
  // element 32 b + 16 vdh + 4 (s % 4).
  const int vs = lane & 15, vdh = (lane >> 4) & 1, tr_r = 4 * half + (vs >> 2);
  uint32_t ktl[DBLK], kth[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) {
    const int unit = 4 * b + 2 * vdh + ((vs & 3) >> 1);
    ktl[b] = uint32_t(tr_r * RB + 16 * (unit ^ swz_k(tr_r)) + 8 * (vs & 1));
    kth[b] = uint32_t((tr_r + 8) * RB + 16 * (unit ^ swz_k(tr_r + 8)) + 8 * (vs & 1));
  }
  // Direct-to-LDS loads: instruction r of wave w fills bytes [1 KB i, 1 KB (i + 1)) of a tile,
  // i = NDMA w + r: lane l unit l % UPR of key row KPI i + l / UPR, from source unit
  // (l % UPR) ^ swz(row).  Keys past the range's end load as zeros.
  uint32_t kdma[NDMA], vdma[NDMA];
#pragma unroll
  for (int r = 0; r < NDMA; ++r) {
    const int row = KPI * (NDMA * w + r) + lane / UPR, u = lane % UPR;
    kdma[r] = uint32_t(row * kv_stride * 2 + 16 * (u ^ swz_k(row)));
    vdma[r] = uint32_t(row * kv_stride * 2 + 16 * (u ^ swz_v(row)));
  }
  const uint32_t lds0 = lds_addr_of(lds);

  const int nA = it.a_end > it.a_start ? (it.a_end - it.a_start + BN - 1) / BN : 0;
  const int nB = it.b_end > it.b_start ? (it.b_end - it.b_start + BN - 1) / BN : 0;
  const int nt = nA + nB;
  auto t_start = [&](int i) { return i < nA ? it.a_start + i * BN : it.b_start + (i - nA) * BN; };
  auto t_end = [&](int i) { return i < nA ? it.a_end : it.b_end; };

  auto issue = [&](int i, int slot) {
    const int start = __builtin_amdgcn_readfirstlane(t_start(i));
    const int keys = __builtin_amdgcn_readfirstlane(min(BN, t_end(i) - start));
    const rsrc_t rk = make_rsrc(K + int64_t(start) * kv_stride + g * D, keys * kv_stride * 2);
    const rsrc_t rv = make_rsrc(V + int64_t(start) * kv_stride + g * D, keys * kv_stride * 2);
    const uint32_t lk = lds0 + slot * 2 * TB + 1024 * NDMA * w;
#pragma unroll
    for (int r = 0; r < NDMA; ++r) buf_load16_lds(rk, lk + 1024 * r, kdma[r]);
#pragma unroll
    for (int r = 0; r < NDMA; ++r) buf_load16_lds(rv, lk + TB + 1024 * r, vdma[r]);
  };

  f32x16_t acc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) acc[b] = f32x16_t{};
  if (nt > 0) issue(0, 0);
  for (int i = 0; i < nt; ++i) {
    const int slot = i & 1;
    // This wave's loads of tile i have landed; after the barrier every wave's have, and every wave
    // has finished tile i - 1, whose slot the next loads overwrite.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (i + 1 < nt) issue(i + 1, slot ^ 1);
    const uint8_t* const kt = lds + slot * 2 * TB;
    const uint8_t* const vt = kt + TB;
    const int start = t_start(i), end = t_end(i);
    const bool causal = i >= nA;
    // Register r of block kb holds key start + 32 kb + 8 (r / 4) + 4 half + r % 4.
    const int lim = (causal ? min(end, row_tok + 1) : end) - start - 4 * half;
    // Only a short tile or one crossing the diagonal needs the mask.  Rows past the item's last
    // token need none: their Q and dO are zero and their lse term 0, so P = 1 and dS = 0.
    const bool masked = end - start < BN || (causal && start + BN - 1 > it.row0);
    // One 32-key block at a time keeps few values live (two workgroups fit on a CU).
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) {
        s = mfma32(load16(kt + 32 * RB * kb + kro[st]), qf[st], s);
        dp = mfma32(load16(vt + 32 * RB * kb + vro[st]), df[st], dp);
      }
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0 = fast_exp2(fmaf(s[r], scale_log2, -l2));
        float p1 = fast_exp2(fmaf(s[r + 1], scale_log2, -l2));
        if (masked) {
          p0 = row_ok && (kb * 32 + 8 * (r >> 2) + (r & 3)) < lim ? p0 : 0.f;
          p1 = row_ok && (kb * 32 + 8 * (r >> 2) + (r & 3) + 1) < lim ? p1 : 0.f;
        }
        pk[r >> 1] = pack_bf16x2(p0 * (dp[r] - dr), p1 * (dp[r + 1] - dr));
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const u32x4_t pv = {pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]};
        const uint8_t* kq = kt + (32 * kb + 16 * m) * RB;
#pragma unroll
        for (int b = 0; b < DBLK; ++b) {
          const u32x2_t lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(kq + ktl[b]));
          const u32x2_t hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(kq + kth[b]));
          acc[b] = mfma32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pv, acc[b]);
        }
      }
    }
  }
  __syncthreads();  // every wave is done with the tiles before the rows are staged over them
  // acc[b] register r holds head-dim element 32 b + 8 (r / 4) + 4 half + r % 4 of this lane's row.
  // The rows go through this wave's part of the (now idle) tile buffers, so that each store
  // instruction writes whole rows (two at d = 128) instead of 32 bytes of each of 32 rows.  Whole
  // lines can take the non-temporal hint (partial lines written that way reach HBM unmerged).
  // Row n at 4D n bytes, its 16-byte unit c at c ^ (n mod 16).
  uint8_t* const stage = lds + w * 32 * 4 * D;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4_t*>(stage + n * 4 * D + 16 * ((8 * b + 2 * j + half) ^ (n & 15))) =
          f32x4_t{acc[b][4 * j], acc[b][4 * j + 1], acc[b][4 * j + 2], acc[b][4 * j + 3]} * scale;
  constexpr int CPR = D / 4;     // 16-byte columns per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int c = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / CPR, rr = w * 32 + r;  // row r of this wave, rr of the item
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + r * 4 * D + 16 * (c ^ (r & 15)));
    if (it.slot < 0) {
      const int tok = it.row0 + rr % TM;
      if (tok < it.row_limit) __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(dQ + (int64_t(tok) * Hq + g * G + rr / TM) * D + 4 * c));
    } else {
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(part_dq + ((int64_t(it.slot) * Hkv + g) * kRowsPerTile + rr) * D + 4 * c));
    }
  }
}

// Sum the split-key dQ partials of one query tile (fixed order).  One thread per (row, 4 elements).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_merge_kernel(float* __restrict__ dQ, const MergeItem* __restrict__ merges,
                                                                const float* __restrict__ part_dq, int Hq, int Hkv,
                                                                int G) {
  constexpr int CH = D / 4;
  constexpr int WG_PER_TILE = kRowsPerTile * CH / 256;
  const int tile = blockIdx.x / WG_PER_TILE, part = blockIdx.x % WG_PER_TILE;
  const int g = tile % Hkv;
  const MergeItem mi = merges[tile / Hkv];
  const int unit = part * 256 + threadIdx.x;
  const int rho = unit / CH, ch = unit % CH;
  const int TM = kRowsPerTile / G;
  const int tok = mi.row0 + rho % TM, h = g * G + rho / TM;
  if (tok >= mi.row_limit) return;
  const int64_t stride = int64_t(Hkv) * kRowsPerTile * D;
  const float* src = part_dq + ((int64_t(mi.slot0) * Hkv + g) * kRowsPerTile + rho) * D + 4 * ch;
  f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int c = 0; c < mi.nslots; ++c) a += *reinterpret_cast<const f32x4_t*>(src + c * stride);  // slot order
  *reinterpret_cast<f32x4_t*>(dQ + (int64_t(tok) * Hq + h) * D + 4 * ch) = a;
}

// MFMA v_mfma_f32_16x16x32_bf16 lane layout: A (16 x 32, M x K): lane l holds A[l % 16][8 (l / 16) + t];
// B (32 x 16, K x N): lane l holds B[8 (l / 16) + t][l % 16]; D (16 x 16): lane l, register r holds
// D[4 (l / 16) + r][l % 16].
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Key-major dK / dV.  A workgroup of four waves takes one item (at most 64 keys of one segment
// and KV head); wave w holds keys k0 + 16 w .. + 15, one per lane column, with their K and V
// fragments (B operands of S = Q K^T and dP = dO V^T) and fp32 dK^T, dV^T accumulators in
// registers.  The rows that read the keys stream through LDS RS (token, head) rows per step
// (token-major, G heads per token), loaded by direct-to-LDS loads into two slots: step i + 1 is
// in flight while step i is computed, with one barrier per step.  Per step and wave:
//   S = Q K^T, dP = dO V^T          rows on M (16-row blocks), keys on N, d as K
//   P = exp2(S scale log2e - lse log2e) on allowed pairs, dS = P (dP - Dr)
//   dV^T += dO^T P, dK^T += Q^T dS  d on M, keys on N, rows as K (32 rows per product), with dO^T
//                                   and Q^T read from LDS by transposing reads
// The 32 rows of one product are, for lane group u = l / 16, rows 4u .. 4u + 3 and 16 + 4u ..
// 16 + 4u + 3 of a 32-row half step: the rows an S register block already holds, so P and dS
// go from the S layout to the B operand without any exchange.
// LDS rows are 2D bytes, 16-byte unit c of row r stored at c ^ swz(r), so that the row reads (16
// rows at one unit) and the transposing reads (8 rows x one unit pair) touch distinct banks.
template <int D, int G>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                             const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                                             const float* __restrict__ nlse2, const float* __restrict__ dvec,
                                                             float* __restrict__ dK, float* __restrict__ dV,
                                                             const KvItem* __restrict__ items, float* __restrict__ part_dkv,
                                                             int Hq, int Hkv, int kv_slots, float scale, float scale_log2) {
  constexpr int RS = 64;                // rows per step
  constexpr int TR = RS / G;            // row tokens per step
  constexpr int RB = 2 * D;             // bytes per row
  constexpr int UPR = D / 8;            // 16-byte units per row
  constexpr int KPI = 1024 / RB;        // rows per direct-to-LDS wave instruction
  constexpr int NDMA = RS / KPI / 4;    // such instructions per wave per tensor per step
  constexpr int KS = D / 32;            // k-steps of S and dP
  constexpr int DB = D / 16;            // 16-wide head-dim blocks of dK^T and dV^T
  constexpr int NRB = RS / 16;          // 16-row blocks per step
  constexpr int TILE = RS * RB;         // bytes per tensor per slot
  static_assert(NDMA >= 1 && NDMA * KPI * 4 == RS, "a step's rows split over four waves");
  __shared__ __align__(1024) uint8_t sq[2][TILE];
  __shared__ __align__(1024) uint8_t sd[2][TILE];
  __shared__ __align__(256) float sl[2][64];  // the rows' -lse log2(e), then their Dr
  __shared__ __align__(256) float sr[2][64];

  const int g = blockIdx.x % Hkv;
  const KvItem it = items[blockIdx.x / Hkv];
  const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, u = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q_stride = Hq * D, kv_stride = Hkv * D;
  const int key = it.k0 + 16 * w + m;  // this lane's key (N index of every product)

  auto swz = [](int r) { return D == 128 ? 2 * (r & 7) + ((r >> 3) & 1) : 2 * ((r >> 1) & 3) + ((r >> 3) & 1); };

  // K and V fragments: lane l holds K[key][32 st + 8 u + t] (B operand of S = Q K^T).
  const int nkeys = it.k_limit - it.k0;
  const rsrc_t rk = make_rsrc(K + int64_t(it.k0) * kv_stride + g * D, nkeys * kv_stride * 2);
  const rsrc_t rv = make_rsrc(V + int64_t(it.k0) * kv_stride + g * D, nkeys * kv_stride * 2);
  const uint32_t k_off = uint32_t(((16 * w + m) * kv_stride + 8 * u) * 2);
  u32x4_t kf[KS], vf[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    kf[st] = buf_load16(rk, k_off + 64 * st);
    vf[st] = buf_load16(rv, k_off + 64 * st);
  }
  // Row reads (A operands of S and dP): row 16 rb + m, unit 4 st + u.
  uint32_t aofs[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) aofs[st] = uint32_t(m * RB + 16 * ((4 * st + u) ^ swz(m)));
  // Transposing reads (A operands of dV^T and dK^T): in lane group u, lane m points at row
  // 4u + m / 4 (+ 16, + 32 j) and head-dim element 16 db + 4 (m % 4), and receives column 16 db + m
  // of rows 4u .. 4u + 3.  Rows + 16 and + 32 leave the swizzle unchanged.
  const int tr_row = 4 * u + (m >> 2);
  uint32_t tofs[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    tofs[db] = uint32_t(tr_row * RB + 16 * ((2 * db + ((m & 3) >> 1)) ^ swz(tr_row)) + 8 * (m & 1));
  // Direct-to-LDS loads: instruction r of wave w fills LDS bytes [1 KB i, 1 KB (i + 1)) of a slot,
  // i = NDMA w + r: rows KPI i .. KPI i + KPI - 1, lane l unit l % UPR of row KPI i + l / UPR from
  // source unit (l % UPR) ^ swz(row).  Row r is token r / G, head g G + r % G of the step.
  uint32_t dofs[NDMA];
#pragma unroll
  for (int r = 0; r < NDMA; ++r) {
    const int row = KPI * (NDMA * w + r) + lane / UPR, c = (lane % UPR) ^ swz(row);
    dofs[r] = uint32_t(((row / G) * q_stride + (row % G) * D) * 2 + 16 * c);
  }
  const uint32_t lofs = uint32_t(((lane / G) * Hq + lane % G) * 4);  // lse / Dr of row `lane`

  f32x4_t ak[DB], av[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    ak[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    av[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // Row steps: the causal range first, then the unmasked one.
  const int nC = it.c1 > it.c0 ? (it.c1 - it.c0 + TR - 1) / TR : 0;
  const int nU = it.u1 > it.u0 ? (it.u1 - it.u0 + TR - 1) / TR : 0;
  const int nS = nC + nU;
  auto step_t0 = [&](int i) { return i < nC ? it.c0 + i * TR : it.u0 + (i - nC) * TR; };
  auto step_end = [&](int i) { return i < nC ? it.c1 : it.u1; };
  // Rows past the range's end load as zeros (Q, dO, -lse log2(e), Dr): their S and dP are 0, so they add
  // P = 1 times a zero dO row to dV and dS = 0 to dK, i.e. nothing.
  auto issue = [&](int i, int slot) {
    const int t0 = __builtin_amdgcn_readfirstlane(step_t0(i));
    const int ntok = __builtin_amdgcn_readfirstlane(min(TR, step_end(i) - t0));
    const int64_t base = (int64_t(t0) * Hq + g * G);
    const rsrc_t bq = make_rsrc(Q + base * D, ntok * q_stride * 2);
    const rsrc_t bd = make_rsrc(dO + base * D, ntok * q_stride * 2);
    const uint32_t lq = lds_addr_of(&sq[slot][0]) + 1024 * NDMA * w, ld = lds_addr_of(&sd[slot][0]) + 1024 * NDMA * w;
#pragma unroll
    for (int r = 0; r < NDMA; ++r) buf_load16_lds(bq, lq + 1024 * r, dofs[r]);
#pragma unroll
    for (int r = 0; r < NDMA; ++r) buf_load16_lds(bd, ld + 1024 * r, dofs[r]);
    if (w == 0) buf_load4_lds(make_rsrc(nlse2 + base, ntok * Hq * 4), lds_addr_of(&sl[slot][0]), lofs);
    if (w == 1) buf_load4_lds(make_rsrc(dvec + base, ntok * Hq * 4), lds_addr_of(&sr[slot][0]), lofs);
  };
  if (nS > 0) issue(0, 0);
  for (int i = 0; i < nS; ++i) {
    const int slot = i & 1;
    // This wave's loads of step i have landed; after the barrier every wave's have, and every wave
    // has finished step i - 1, whose slot the next loads overwrite.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (i + 1 < nS) issue(i + 1, slot ^ 1);
    const int t0 = step_t0(i);
    // Causal steps whose first token is at or after the last key read every key: no mask.
    const bool masked = i < nC && t0 < it.k_limit - 1;
    const uint8_t* qs = &sq[slot][0];
    const uint8_t* ds = &sd[slot][0];
#pragma unroll
    for (int hs = 0; hs < NRB / 2; ++hs) {  // 32-row half steps
      f32x4_t s[2], dp[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int rb = 2 * hs + b;
        s[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dp[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          s[b] = mfma16(load16(qs + aofs[st] + 16 * RB * rb), kf[st], s[b]);
          dp[b] = mfma16(load16(ds + aofs[st] + 16 * RB * rb), vf[st], dp[b]);
        }
      }
      // Register r of block b holds row 32 hs + 16 b + 4 u + r of the step, for this lane's key.
      uint32_t pp[4], pd[4];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int r0 = 32 * hs + 16 * b + 4 * u;
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(&sl[slot][r0]);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&sr[slot][r0]);
        float pr[4], dsv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = fast_exp2(fmaf(s[b][r], scale_log2, l4[r]));
          if (masked) pr[r] = key <= t0 + (r0 + r) / G ? pr[r] : 0.f;
          dsv[r] = pr[r] * (dp[b][r] - d4[r]);
        }
        pp[2 * b] = pack_bf16x2(pr[0], pr[1]);
        pp[2 * b + 1] = pack_bf16x2(pr[2], pr[3]);
        pd[2 * b] = pack_bf16x2(dsv[0], dsv[1]);
        pd[2 * b + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      const u32x4_t bp = {pp[0], pp[1], pp[2], pp[3]};
      const u32x4_t bd = {pd[0], pd[1], pd[2], pd[3]};
      const uint32_t hrow = 32 * RB * hs;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint8_t* dpt = ds + hrow + tofs[db];  // rows 4u .. 4u + 3; + 16 RB: rows 16 + 4u ..
        const uint8_t* qpt = qs + hrow + tofs[db];
        const u32x2_t dlo = lds_read_tr16(reinterpret_cast<const uint16_t*>(dpt));
        const u32x2_t dhi = lds_read_tr16(reinterpret_cast<const uint16_t*>(dpt + 16 * RB));
        av[db] = mfma16(u32x4_t{dlo[0], dlo[1], dhi[0], dhi[1]}, bp, av[db]);
        const u32x2_t qlo = lds_read_tr16(reinterpret_cast<const uint16_t*>(qpt));
        const u32x2_t qhi = lds_read_tr16(reinterpret_cast<const uint16_t*>(qpt + 16 * RB));
        ak[db] = mfma16(u32x4_t{qlo[0], qlo[1], qhi[0], qhi[1]}, bd, ak[db]);
      }
    }
  }
  __syncthreads();  // every wave is done with the last step's rows before they are overwritten
  // ak / av[db] register r holds head-dim element 16 db + 4 u + r of this lane's key.  The fp32
  // rows go through this wave's part of the idle row slots (dK^T in sq, dV^T in sd), so that each
  // store writes whole rows.  Key row n at 4 D n bytes, its 16-byte unit c at c ^ (n mod 16).
  uint8_t* const stk = &sq[0][0] + w * 16 * 4 * D;
  uint8_t* const stv = &sd[0][0] + w * 16 * 4 * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int o = m * 4 * D + 16 * ((4 * db + u) ^ m);
    *reinterpret_cast<f32x4_t*>(stk + o) = ak[db] * scale;
    *reinterpret_cast<f32x4_t*>(stv + o) = av[db];
  }
  constexpr int CPR = D / 4;     // 16-byte columns per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int c = lane % CPR;
#pragma unroll
  for (int i = 0; i < 16 / RPI; ++i) {
    const int r = RPI * i + lane / CPR, kk = 16 * w + r;
    if (it.k0 + kk >= it.k_limit) continue;
    const int o = r * 4 * D + 16 * (c ^ r);
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(stk + o);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(stv + o);
    float *pk_, *pv_;
    if (it.slot < 0) {
      pk_ = dK + (int64_t(it.k0 + kk) * Hkv + g) * D;
      pv_ = dV + (int64_t(it.k0 + kk) * Hkv + g) * D;
    } else {
      const int64_t base = ((int64_t(it.slot) * Hkv + g) * kBwdKeyTile + kk) * D;
      pk_ = part_dkv + base;
      pv_ = part_dkv + int64_t(kv_slots) * Hkv * kBwdKeyTile * D + base;
    }
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(pk_ + 4 * c));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(pv_ + 4 * c));
  }
}

// Sum the split dK / dV partials of one key tile (fixed order).  One thread per (key, 4 elements).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkv_merge_kernel(float* __restrict__ dK, float* __restrict__ dV,
                                                                 const KvMerge* __restrict__ merges,
                                                                 const float* __restrict__ part_dkv, int Hkv,
                                                                 int kv_slots) {
  constexpr int CH = D / 4;
  constexpr int WG_PER_TILE = kBwdKeyTile * CH / 256;
  const int tile = blockIdx.x / WG_PER_TILE, part = blockIdx.x % WG_PER_TILE;
  const int g = tile % Hkv;
  const KvMerge mi = merges[tile / Hkv];
  const int unit = part * 256 + threadIdx.x;
  const int kk = unit / CH, ch = unit % CH;
  const int key = mi.k0 + kk;
  if (key >= mi.k_limit) return;
  const int64_t stride = int64_t(Hkv) * kBwdKeyTile * D;
  const float* src = part_dkv + ((int64_t(mi.slot0) * Hkv + g) * kBwdKeyTile + kk) * D + 4 * ch;
  const float* srcv = src + int64_t(kv_slots) * stride;
  f32x4_t a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int c = 0; c < mi.nslots; ++c) {  // slot order
    a += *reinterpret_cast<const f32x4_t*>(src + c * stride);
    b += *reinterpret_cast<const f32x4_t*>(srcv + c * stride);
  }
  *reinterpret_cast<f32x4_t*>(dK + (int64_t(key) * Hkv + g) * D + 4 * ch) = a;
  *reinterpret_cast<f32x4_t*>(dV + (int64_t(key) * Hkv + g) * D + 4 * ch) = b;
}

template <int D, int G>
static hipError_t launch_bwd_t(const BwdLaunch& a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (a.n_items > 0) {
    attn_bwd_dq_kernel<D, G><<<unsigned(a.n_items * a.num_kv_heads), 256, 0, stream>>>(
        a.Q, a.K, a.V, a.O, a.dO, a.lse, a.dvec, a.nlse2, a.dQ, a.items, a.part_dq, a.num_q_heads, a.num_kv_heads, a.scale,
        a.scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_merges > 0) {
    attn_bwd_dq_merge_kernel<D><<<unsigned(a.n_merges * a.num_kv_heads * (kRowsPerTile * (D / 4) / 256)), 256, 0,
                                  stream>>>(a.dQ, a.merges, a.part_dq, a.num_q_heads, a.num_kv_heads, G);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_kv_items > 0) {
    attn_bwd_dkv_kernel<D, G><<<unsigned(a.n_kv_items * a.num_kv_heads), 256, 0, stream>>>(
        a.Q, a.K, a.V, a.dO, a.nlse2, a.dvec, a.dK, a.dV, a.kv_items, a.part_dkv, a.num_q_heads, a.num_kv_heads,
        a.kv_slots, a.scale, a.scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_kv_merges > 0) {
    attn_bwd_dkv_merge_kernel<D><<<unsigned(a.n_kv_merges * a.num_kv_heads * (kBwdKeyTile * (D / 4) / 256)), 256,
                                   0, stream>>>(a.dK, a.dV, a.kv_merges, a.part_dkv, a.num_kv_heads, a.kv_slots);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_attn_bwd(const BwdLaunch& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (a.head_dim == 128) {
    switch (G) {
      case 1: return launch_bwd_t<128, 1>(a, stream);
      case 2: return launch_bwd_t<128, 2>(a, stream);
      case 4: return launch_bwd_t<128, 4>(a, stream);
      default: return launch_bwd_t<128, 8>(a, stream);
    }
  }
  switch (G) {
    case 1: return launch_bwd_t<64, 1>(a, stream);
    case 2: return launch_bwd_t<64, 2>(a, stream);
    case 4: return launch_bwd_t<64, 4>(a, stream);
    default: return launch_bwd_t<64, 8>(a, stream);
  }
}

}  // namespace br
