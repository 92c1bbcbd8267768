// Block-sparse prefill attention for BlockRank prompts on gfx950 (MI355X).
//
// Computes softmax(Q K^T * scale + M) V where M allows: instruction rows -> instruction keys
// causally; document rows -> the whole instruction plus their own document causally; final
// query rows -> everything before the query plus the query causally (BlockRank summary,
// section 3.4 "Blockwise Structured Attention"; blog, block mask with causal diagonal blocks C;
// BlockSearch section 3.2 for the causal reading of the diagonal blocks).  The host plan lists
// only allowed (row tile, key range) pairs; this kernel never visits a forbidden block.
//
// Row token indices address Q, O and lse relative to q_row_base (0 for whole prompts; the corpus
// length when only query rows over a cached corpus are computed).
//
// Work item = 128 (token, head) rows: TM = 128 / G consecutive tokens of the G query heads
// that share one KV head (grouped-query packing), so each K/V tile staged in LDS serves G
// heads.  Rows are token-major (row 32 w + n of wave w is token (32 w + n) / G, head
// (32 w + n) % G), so wave w owns 32 / G whole tokens; a wave whose tokens all lie past an
// item's last token (the short last row tile of a document) skips that item's arithmetic.
// Keys are visited in tiles of 32:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16 with keys on M and query rows on N, so each lane
//                 holds one query row and 16 of the tile's keys; the row max needs one
//                 cross-half exchange (v_permlane32_swap);
//   online softmax in fp32 (log2 domain, exp2) with lazy rescaling of the accumulator;
//   O^T += V^T P^T with P rounded to bf16; the transposed V fragments come from transposing
//                 LDS reads (ds_read_b64_tr_b16).
//
// Software pipeline.  The kernel is persistent: each workgroup serves one KV head and walks the
// key tiles of its share of the item list (a host list schedule) as one flat sequence that runs
// across item boundaries.  Iteration j of a wave issues
//   the P.V products of tile j-1, the S^T products of tile j+1        (matrix cores)
//   the softmax of tile j                                                (vector ALU)
// so the exponentials of one tile overlap the matrix products of its neighbours.  K and V tiles
// go from memory straight into LDS (buffer loads with the LDS flag: no register staging) through
// rings of NS slots, NS - 1 tiles ahead of use; one wait for the wave's own loads plus one
// barrier per tile publishes them.  The next item's Q fragments are loaded into registers while
// the current item runs.  Loads use buffer resources sized to the valid rows: rows past a range
// end read as zero, and output rows past a tile's last token are dropped by the hardware.
// Output rows are staged through the wave's own part of the Q buffer (between reading one
// item's Q fragments and loading the next item's rows) so each store writes whole 128-byte
// lines (stores of 32 bytes per row were measured to cost about a sixth of the kernel time),
// with the non-temporal hint, which leaves the L2 to the K/V tiles that are re-read.
//
// LDS layouts (16-byte units, XOR-swizzled instead of padded, because a direct-to-LDS load
// fills 1 KB of consecutive LDS per wave instruction):
//   K tile: row k at k * D * 2 bytes, unit c of the row stored at unit c ^ swz_k(k), so the 16
//           keys a quarter-wave reads at one unit fall in 16 different bank groups;
//   V tile: unit c of row k at unit c ^ swz_v(k), so a half-wave's transposing read (4 keys x 4
//           units) touches 16 different bank groups.
// Q fragments use a permutation of the head dimension inside each 16-wide MFMA step: with
// H = D/32, k-step st of lane half h takes unit (st % H) + H h + 2H (st / H) of a row, so a lane
// holds units u and u + D/16 (elements e and e + D/2) together; the K fragments are read with the
// same permutation, and the contraction over d is unchanged.  Holding both halves of a row lets
// the rotary embedding be applied to Q in registers: pairs (e, e + D/2) in the split layout, and
// pairs inside a unit in the adjacent layout (the ROPE variants of the kernel).
//
// Query rows of long prompts are split over key chunks; their fp32 partials (m, l, o) are
// combined by attn_merge_kernel.
#include <type_traits>

#include "attn_merge.h"
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace br {

// Accumulator rescaling is skipped until the running maximum grows by more than this many
// log2 units, so probabilities stay <= 2^8 before normalisation (exact in fp32 and bf16 range).
constexpr float kRescaleSlack = 8.0f;
constexpr int kFwdKeys = 32;   // keys per LDS tile
constexpr int kFwdSlots = 3;   // tiles per ring (K ring and V ring): loads run two tiles ahead

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding), then a workgroup
// barrier.  The asm statement also keeps the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(N) alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (min(n, 63) >> 2) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<4>(); break;
    case 2: wait_vm<8>(); break;
    case 3: wait_vm<12>(); break;
    case 4: wait_vm<16>(); break;
    case 5: wait_vm<20>(); break;
    case 6: wait_vm<24>(); break;
    case 7: wait_vm<28>(); break;
    case 8: wait_vm<32>(); break;
    case 9: wait_vm<36>(); break;
    case 10: wait_vm<40>(); break;
    case 11: wait_vm<44>(); break;
    case 12: wait_vm<48>(); break;
    case 13: wait_vm<52>(); break;
    case 14: wait_vm<56>(); break;
    default: wait_vm<60>(); break;
  }
}

// The same with a barrier after the wait.
__device__ __forceinline__ void wait_vm_barrier_dyn(int n) {
  switch (min(n, 63) >> 2) {
    case 0: wait_vm_barrier<0>(); break;
    case 1: wait_vm_barrier<4>(); break;
    case 2: wait_vm_barrier<8>(); break;
    case 3: wait_vm_barrier<12>(); break;
    case 4: wait_vm_barrier<16>(); break;
    case 5: wait_vm_barrier<20>(); break;
    case 6: wait_vm_barrier<24>(); break;
    case 7: wait_vm_barrier<28>(); break;
    case 8: wait_vm_barrier<32>(); break;
    case 9: wait_vm_barrier<36>(); break;
    case 10: wait_vm_barrier<40>(); break;
    case 11: wait_vm_barrier<44>(); break;
    case 12: wait_vm_barrier<48>(); break;
    case 13: wait_vm_barrier<52>(); break;
    case 14: wait_vm_barrier<56>(); break;
    default: wait_vm_barrier<60>(); break;
  }
}

// ROPE: 0 Q is used as given; 1 or 2 each item's Q rows are rotated after they are read (split
// or adjacent pairs) with cos/sin from `rope_cs` ([table row][D/2 pairs][cos, sin] fp32), the
// item's first token at table row item_pidx[item] and its later tokens at the rows after it.
template <int D, int G, int NS, int ROPE>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                       float* __restrict__ lse, const AttnItem* __restrict__ items,
                                                       const int32_t* __restrict__ ranges, float* __restrict__ part_o,
                                                       float* __restrict__ part_ml, int Hq, int Hkv, float scale_log2,
                                                       int q_row_base, float sink_log2,
                                                       const float* __restrict__ rope_cs,
                                                       const int32_t* __restrict__ item_pidx) {
  constexpr int TM = kRowsPerTile / G;  // tokens per item
  constexpr int BN = kFwdKeys;
  constexpr int RB = 2 * D;             // bytes per row of one head
  constexpr int TB = BN * RB;           // bytes per K or V tile
  constexpr int UPR = D / 8;            // 16-byte units per row
  constexpr int DSTEPS = D / 16;        // MFMA k-steps over the head dimension
  constexpr int DBLK = D / 32;          // 32-wide output blocks over the head dimension
  constexpr int KPI = 1024 / RB;        // key rows per direct-to-LDS wave instruction
  constexpr int NDMA = BN / KPI / 4;    // such instructions per wave per tile, for K and for V
  constexpr int LOADS = 2 * NDMA;       // vector-memory loads a wave issues per iteration
  constexpr int WIN = 6;                // descriptor window = loop unroll factor
  static_assert(NDMA >= 1 && NDMA * KPI * 4 == BN, "tile split over four waves");
  static_assert(NS == 3, "the loop below is unrolled for three ring slots and two register sets");
  static_assert(DSTEPS * KPI == 32, "one wave's Q rows in DSTEPS direct-to-LDS instructions");

  __shared__ __align__(1024) uint8_t vring[NS][TB];
  __shared__ __align__(1024) uint8_t kring[NS][TB];
  __shared__ __align__(1024) uint8_t qbuf[kRowsPerTile * RB];  // an item's Q rows (wave w: rows 32w..)

  const int g = blockIdx.x % Hkv;
  const int wg = blockIdx.x / Hkv;
  const int it_begin = ranges[wg], it_end = ranges[wg + 1];
  if (it_begin >= it_end) return;  // uniform per workgroup

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, half = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int rho = w * 32 + n;  // this lane's row within the item
  const int tt = rho / G, hh = rho % G;  // token-major: a token's G heads are adjacent rows
  const int h = g * G + hh;
  const int q_stride = Hq * D, kv_stride = Hkv * D;  // elements between consecutive tokens

  // ---- swizzles (16-byte units within a row) ----
  auto swz_k = [](int k) { return D == 128 ? (k & 15) : ((k >> 1) & 7); };
  auto swz_v = [](int k) { return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); };

  // LDS byte addresses (M0 values of the direct-to-LDS loads): this wave's share of each ring slot.
  const uint32_t k_lds = lds_addr_of(kring) + 1024 * NDMA * w;
  const uint32_t v_lds = lds_addr_of(vring) + 1024 * NDMA * w;
  const uint32_t q_lds = lds_addr_of(qbuf) + 32 * RB * w;
  // K fragment of k-step st for this lane: key n, unit qunit(st) (the head-dim permutation).
  constexpr int HU = DSTEPS / 2;  // units of each half of the head dimension held by one lane
  auto qunit = [&](int st) { return (st % HU) + HU * half + 2 * HU * (st / HU); };
  uint32_t kofs[DSTEPS];
#pragma unroll
  for (int st = 0; st < DSTEPS; ++st) kofs[st] = uint32_t(n * RB + 16 * (qunit(st) ^ swz_k(n)));
  // Transposing V reads: in each 16-lane group (s = lane % 16, head-dim half dh = (lane / 16) % 2)
  // lane s points at key 4 half + s / 4 and head-dim element 16 dh + 4 (s % 4) of a 32-wide block;
  // keys 16 m (+8) shift the row by a multiple of 8, which leaves the swizzle unchanged.
  const int vs = lane & 15, vdh = (lane >> 4) & 1;
  const int vkey = 4 * half + (vs >> 2);
  uint32_t vofs[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
    vofs[b] = uint32_t(vkey * RB + 16 * ((4 * b + 2 * vdh + ((vs & 3) >> 1)) ^ swz_v(vkey)) + 8 * (vs & 1));
  // Direct-to-LDS loads: wave instruction r of this wave fills LDS bytes [i KB, (i + 1) KB) of a
  // tile, i = NDMA w + r, i.e. key rows KPI i .. KPI i + KPI - 1; lane l fills unit l % UPR of
  // row KPI i + l / UPR with source unit (l % UPR) ^ swz(row).
  uint32_t kdma[NDMA], vdma[NDMA];
#pragma unroll
  for (int r = 0; r < NDMA; ++r) {
    const int key = KPI * (NDMA * w + r) + lane / UPR, u = lane % UPR;
    kdma[r] = uint32_t(key * kv_stride * 2 + 16 * (u ^ swz_k(key)));
    vdma[r] = uint32_t(key * kv_stride * 2 + 16 * (u ^ swz_v(key)));
  }

  // ---- the flat tile sequence ----
  // A tile is {first key, (item << 9) | (keys << 3) | flags, first row of its item}: keys =
  // valid keys of the tile (1..32); flags 1 causal range, 2 first tile of its item, 4 last tile
  // of its item.  Items past it_end are "no tile": nothing to read, and they count as one-tile
  // items so that the stages around them reset cleanly.
  constexpr int F_CAUSAL = 1, F_FIRST = 2, F_LAST = 4, F_IDLE = 512, IT_SHIFT = 10;
  auto code_it = [](int code) { return code >> IT_SHIFT; };
  auto code_keys = [](int code) { return (code >> 3) & 63; };
  auto n_tiles = [](int a0, int a1) { return a1 > a0 ? (a1 - a0 + BN - 1) / BN : 0; };
  // Lead cursor: item c_it; its next tile starts at key c_cur of the range ending at c_end; c_left
  // tiles of the item are left, c_la of them in the unmasked range; c_base holds the item's code
  // bits (index, idle), c_fl the range and first-tile flags of the next tile.
  int c_it = it_begin, c_cur, c_end, c_left, c_la, c_base, c_fl, c_row0, c_b0, c_b1;
  const int w_tok0 = 32 * w / G;  // first token of this wave's rows
  auto load_item = [&]() {
    if (c_it < it_end) {
      const AttnItem it = items[c_it];
      const int na = n_tiles(it.a_start, it.a_end);
      c_row0 = it.row0;
      c_base = (c_it << IT_SHIFT) | (w_tok0 >= it.row_limit - it.row0 ? F_IDLE : 0);
      c_la = na;
      c_left = na + n_tiles(it.b_start, it.b_end);
      c_cur = na > 0 ? it.a_start : it.b_start;
      c_end = na > 0 ? it.a_end : it.b_end;
      c_fl = F_FIRST | (na > 0 ? 0 : F_CAUSAL);
      c_b0 = it.b_start;
      c_b1 = it.b_end;
    }
  };
  load_item();
  auto take = [&](int& start, int& code, int& row0) {
    if (c_it >= it_end) {
      start = row0 = 0;
      code = (it_end << IT_SHIFT) | F_FIRST | F_LAST | F_IDLE;
      return;
    }
    start = c_cur;
    code = c_base | c_fl | (min(BN, c_end - c_cur) << 3) | (c_left == 1 ? F_LAST : 0);
    row0 = c_row0;
    c_fl &= ~F_FIRST;
    c_cur += BN;
    if (--c_la == 0) {  // the unmasked range is done: the causal range follows
      c_cur = c_b0;
      c_end = c_b1;
      c_fl = F_CAUSAL;
    }
    if (--c_left == 0) {
      ++c_it;
      load_item();
    }
  };
  int n_total = 0;
  for (int i = it_begin; i < it_end; ++i) {
    const int4 rg = *reinterpret_cast<const int4*>(&items[i].a_start);  // a_start, a_end, b_start, b_end
    n_total += n_tiles(rg.x, rg.y) + n_tiles(rg.z, rg.w);
  }

  // ---- loads ----
  // One resource per tensor based at this KV head's column; a tile is addressed by the scalar
  // offset start * kv_stride * 2 and bounded by a record count that ends at its last valid key, so
  // key rows past a range end read as zero (the host keeps K and V under 4 GB).
  const uint16_t* const k_base = K + g * D;
  const uint16_t* const v_base = V + g * D;
  auto issue_k = [&](int start, int code, int slot) {  // "no tile" has start 0 and no keys
    start = __builtin_amdgcn_readfirstlane(start);  // uniform: keeps the offsets in scalar registers
    code = __builtin_amdgcn_readfirstlane(code);
    const uint32_t s0 = uint32_t(start) * uint32_t(kv_stride * 2);
    const uint32_t end = s0 + uint32_t(code_keys(code)) * uint32_t(kv_stride * 2);
    const rsrc_t r = make_rsrc(k_base, int(end));
#pragma unroll
    for (int i = 0; i < NDMA; ++i) buf_load16_lds(r, k_lds + slot * TB + 1024 * i, kdma[i], s0);
  };
  auto issue_v = [&](int start, int code, int slot) {  // "no tile" has start 0 and no keys
    start = __builtin_amdgcn_readfirstlane(start);
    code = __builtin_amdgcn_readfirstlane(code);
    const uint32_t s0 = uint32_t(start) * uint32_t(kv_stride * 2);
    const uint32_t end = s0 + uint32_t(code_keys(code)) * uint32_t(kv_stride * 2);
    const rsrc_t r = make_rsrc(v_base, int(end));
#pragma unroll
    for (int i = 0; i < NDMA; ++i) buf_load16_lds(r, v_lds + slot * TB + 1024 * i, vdma[i], s0);
  };
  // Resource over an item's valid rows of a [T, Hq, D] tensor, based at its first row and head.
  auto row_rsrc = [&](const uint16_t* base, int row0, int row_limit) {
    const int rows = min(TM, row_limit - row0);
    return make_rsrc(base + (int64_t(row0 - q_row_base) * Hq + g * G) * D, rows * q_stride * 2);
  };
  // Q rows of an item go to qbuf with direct-to-LDS loads (each wave its own 32 rows, laid out and
  // swizzled like a K tile), then into the fragments `qf` (B operand of S^T, the head-dim
  // permutation of the K fragments).  Each wave reads back only rows it loaded itself, so its own
  // vector-memory wait suffices and no barrier is involved.
  u32x4_t qf[DSTEPS];
  // Per-lane source offsets of the Q loads: DSTEPS instructions of KPI rows cover the wave's 32 rows.
  uint32_t qdma[DSTEPS];
#pragma unroll
  for (int i = 0; i < DSTEPS; ++i) {
    const int rq = KPI * i + lane / UPR, u = lane % UPR, rr = 32 * w + rq;
    qdma[i] = uint32_t(((rr / G) * q_stride + (rr % G) * D) * 2 + 16 * (u ^ swz_k(rq)));
  }
  auto issue_q = [&](int it) {
    rsrc_t r = make_rsrc(Q, 0);
    if (it < it_end) {
      const int2 rr = *reinterpret_cast<const int2*>(&items[it].row0);
      r = row_rsrc(Q, rr.x, rr.y);
    }
#pragma unroll
    for (int i = 0; i < DSTEPS; ++i) buf_load16_lds_nt(r, q_lds + 1024 * i, qdma[i]);
  };

  // ---- pipeline state ----
  f32x16_t o[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) o[b] = f32x16_t{};
  f32x16_t sb[2] = {f32x16_t{}, f32x16_t{}};  // S^T of tiles j (sb[(j + 1) & 1]) and j + 1
  uint32_t pk[8];  // bf16 P: of tile j - 1 until its P.V products have read it, then of tile j
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = 0u;
  float m_run = -INFINITY, l_run = 0.f, m_prev = -INFINITY, l_prev = 0.f;

  // Descriptor window: tile t at index (t + 1) mod WIN; iteration j uses tiles j - 1 .. j + NS.
  int d_start[WIN], d_code[WIN], d_row0[WIN];
#pragma unroll
  for (int k = 0; k < WIN; ++k) {
    d_start[k] = d_row0[k] = 0;
    d_code[k] = (it_end << IT_SHIFT) | F_FIRST | F_LAST | F_IDLE;  // tiles -2 and -1: none
  }
#pragma unroll
  for (int t = 0; t < NS; ++t) take(d_start[t + 1], d_code[t + 1], d_row0[t + 1]);  // tiles 0 .. NS - 1

  // Prologue: the first item's Q (iteration -1 reads it into qf), then the loads of virtual
  // iterations j = -NS .. -2, each issuing K of tile j + NS and V of tile j + NS - 2 (none for
  // negative tiles: zero-size loads that still write zeros, so every slot is initialised).
  issue_q(it_begin);
#pragma unroll
  for (int jv = -NS; jv <= -2; ++jv) {
    const int kt = jv + NS, vt = jv + NS - 2;
    issue_k(d_start[kt + 1], d_code[kt + 1], kt % NS);
    const int vi = vt >= 0 ? vt + 1 : 0;
    issue_v(d_start[vi], d_code[vi], (jv - 2 + 2 * NS) % NS);
  }
  // Vector-memory operations issued after the last Q batch that always issue (for the wait before
  // its rows are read): the prologue's K/V loads.
  int since_q = (NS - 1) * LOADS;
  // Q buffer state: 0 the next item's rows are loading (or loaded); 1 read this iteration, the
  // epilogue of the item before runs next iteration through the buffer; 2 free, load item q_next.
  int q_state = 0, q_next = 0;
  // Unconditional vector-memory operations (Q batches, output stores) that iterations j - 1 and
  // j - 2 issued after their K/V loads.
  int ex_prev = 0, ex_prev2 = 0;
  // Row range and partial slot of the item whose last P.V products run in the next iteration.
  int e_row0 = 0, e_row_limit = 0, e_slot = -1;

  // ---- one pipeline iteration (PH = (j + 1) mod WIN, compile-time) ----
  auto iteration = [&](auto ph_tag) {
    constexpr int PH = decltype(ph_tag)::value;
    constexpr int KSLOT_LOAD = (PH + NS - 1) % NS;  // slot of K tile j + NS  (= j mod NS)
    constexpr int VSLOT_LOAD = (PH + NS - 3) % NS;  // slot of V tile j + NS - 2
    constexpr int KSLOT_S = PH % NS;                 // slot of K tile j + 1
    constexpr int VSLOT_PV = (PH + NS - 2) % NS;     // slot of V tile j - 1
    constexpr int CUR = PH & 1, NXT = CUR ^ 1;       // S^T register sets of tiles j and j + 1
    // Window index of tile j + k is (PH + k) mod WIN.
    constexpr int IP = (PH + WIN - 1) % WIN, IC = PH, IS = (PH + 1) % WIN;  // tiles j - 1, j, j + 1
    constexpr int IK = (PH + NS) % WIN, IV = (PH + NS - 2) % WIN;           // tiles j + NS, j + NS - 2
    constexpr int INEW = (PH + NS + 1) % WIN;                                 // tile j + NS + 1
    f32x16_t& s_cur = sb[CUR];
    f32x16_t& s_nxt = sb[NXT];

    // 1. K of tile j + 1 and V of tile j - 1 have landed in every wave: they were issued in
    // iteration j + 1 - NS (= j - 2); after them came that iteration's extra operations, the K/V
    // loads of iteration j - 1 and its extra operations (vector-memory operations complete in
    // issue order on gfx9, stores included).
    {
      const int x = ex_prev + ex_prev2;
      if (x == 0)
        wait_vm_barrier<(NS - 2) * LOADS>();
      else
        wait_vm_barrier_dyn((NS - 2) * LOADS + x);
      ex_prev2 = ex_prev;
      ex_prev = 0;
    }
    // 2. Loads NS - 1 tiles ahead: K of tile j + NS, V of tile j + NS - 2.
    issue_k(d_start[IK], d_code[IK], KSLOT_LOAD);
    issue_v(d_start[IV], d_code[IV], VSLOT_LOAD);
    since_q += LOADS;
    // 3. Tile j + 1 starts an item: read its Q fragments.  Its Q rows were loaded after the
    // previous epilogue; when that epilogue has not happened yet (the item before is a single
    // tile), load them now.
    const int s_code = d_code[IS];
    if ((s_code & F_FIRST) && code_it(s_code) < it_end) {
      if (q_state != 0) {
        issue_q(code_it(s_code));
        since_q = 0;
        ex_prev += DSTEPS;
      }
      wait_vm_dyn(since_q);  // the Q batch (and everything older) has landed
      // The wave's Q region offset is made opaque here so that the compiler forms these
      // addresses when needed instead of keeping eight more registers live across the loop.
      uint32_t qw = uint32_t(32 * RB) * uint32_t(w);
      asm volatile("" : "+s"(qw));
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) qf[st] = *reinterpret_cast<const u32x4_t*>(&qbuf[qw + kofs[st]]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the buffer is reused
      if constexpr (ROPE != 0) {
        // This lane's token: cos/sin of its table row, then the rotation of qf in registers, with
        // the arithmetic of the separate rotation kernel (fp32, rounded once to bf16).
        const float* tr = rope_cs + int64_t(item_pidx[code_it(s_code)] + tt) * D;
#pragma unroll
        for (int st = 0; st < (ROPE == 1 ? HU : DSTEPS); ++st) {
          const int u = qunit(st);
          if constexpr (ROPE == 1) {
            // units u (elements 8u..8u+7) and u + D/16 hold the pairs 8u .. 8u+7
            const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(tr + 16 * u);
            const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(tr + 16 * u + 4);
            const f32x4_t c2 = *reinterpret_cast<const f32x4_t*>(tr + 16 * u + 8);
            const f32x4_t c3 = *reinterpret_cast<const f32x4_t*>(tr + 16 * u + 12);
            const float cs[8] = {c0[0], c0[2], c1[0], c1[2], c2[0], c2[2], c3[0], c3[2]};
            const float sn[8] = {c0[1], c0[3], c1[1], c1[3], c2[1], c2[3], c3[1], c3[3]};
            rope_rotate_split8(qf[st], qf[st + HU], cs, sn);
          } else {
            // unit u holds the pairs 4u .. 4u+3
            const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(tr + 8 * u);
            const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(tr + 8 * u + 4);
            const float cs[4] = {c0[0], c0[2], c1[0], c1[2]};
            const float sn[4] = {c0[1], c0[3], c1[1], c1[3]};
            rope_rotate_adjacent4(qf[st], cs, sn);
          }
        }
      }
      q_state = 1;
      q_next = code_it(s_code) + 1;
    }
    // 4. Softmax of tile j, part 1: mask.
    const int c_code = d_code[IC], c_start = d_start[IC], c_row0 = d_row0[IC];
    const int c_keys = code_keys(c_code);
    const bool c_valid = code_it(c_code) < it_end;
    const bool c_first = (c_code & F_FIRST) != 0;
    const bool c_causal = (c_code & F_CAUSAL) != 0;
    if (c_first) {
      m_prev = m_run;
      l_prev = l_run;
    }
    // Tiles j - 1, j and j + 1 all belong to items where this wave has no valid rows: skip the
    // arithmetic (the loads, waits and barriers above still run).
    const bool idle3 = (d_code[IP] & d_code[IC] & d_code[IS] & F_IDLE) != 0;
    if (!idle3) {
      if (!c_valid || c_keys < BN || (c_causal && c_start + BN - 1 > c_row0)) {
        // Register r holds key start + 8 (r / 4) + 4 half + r % 4.
        const int lim = (c_valid ? (c_causal ? min(c_keys, c_row0 + tt + 1 - c_start) : c_keys) : 0) - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r) s_cur[r] = (8 * (r >> 2) + (r & 3)) < lim ? s_cur[r] : -INFINITY;
      }

      // 5. Matrix products of tiles j - 1 (P.V) and j + 1 (S^T), softmax of tile j, in three phases
      // separated by scheduling fences, each pairing matrix-core work with independent vector work:
      //   A  P.V MFMAs of tile j - 1, keys 0..15    | row maximum of tile j
      //   B  P.V MFMAs of tile j - 1, keys 16..31   | exponentials of keys whose P slots A freed
      //   C  S^T MFMAs of tile j + 1                | remaining exponentials, row sum
      // Each phase's LDS operands are read one phase ahead.  P of tile j overwrites P of tile j - 1
      // in the registers the P.V products have finished reading.  In phases A and B each product
      // is followed by two of the next phase's LDS reads and a few vector instructions
      // (scheduling groups), so a wave's in-order issue does not wait on a busy matrix core with
      // independent work behind it.  The wave raises its issue priority for the three phases:
      // when both waves of a SIMD can issue, the one with matrix work goes first.
      const uint8_t* vt_base = &vring[VSLOT_PV][0];
      const uint8_t* kt_base = &kring[KSLOT_S][0];
      u32x4_t vf[2][DBLK];
      auto read_v = [&](int m) {
#pragma unroll
        for (int b = 0; b < DBLK; ++b) {
          const uint16_t* vp = reinterpret_cast<const uint16_t*>(vt_base + vofs[b] + 16 * m * RB);
          const u32x2_t lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 8 * D);
          vf[m][b] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
      };
      u32x4_t kf[DSTEPS];
      float lsum0 = 0.f, lsum1 = 0.f;  // two partial row sums shorten the add chain
      float mu = 0.f;
      // Exponentials of s_cur registers [r0, r1) (pairs), packed into pk[r / 2].
      auto exps = [&](int r0, int r1) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          if (r < r0 || r >= r1) continue;
          const float p0 = fast_exp2(fmaf(s_cur[r], scale_log2, -mu));
          const float p1 = fast_exp2(fmaf(s_cur[r + 1], scale_log2, -mu));
          pk[r >> 1] = pack_bf16x2(p0, p1);
          if (r & 2)
            lsum1 += p0 + p1;
          else
            lsum0 += p0 + p1;
        }
      };
      constexpr int R_B = 6;  // exponentials of registers [0, R_B) in phase B, the rest in C
      read_v(0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      // Phase A.
      {
        const u32x4_t pv = {pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int b = 0; b < DBLK; ++b) o[b] = mfma32(vf[0][b], pv, o[b]);
      }
      read_v(1);
      float mt = fmaxf(fmaxf(s_cur[0], s_cur[1]), s_cur[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mt = fmaxf(fmaxf(mt, s_cur[r]), s_cur[r + 1]);
      mt = fmaxf(mt, s_cur[15]);
      mt = max_halves(mt) * scale_log2;
      const bool need = !c_first && mt > m_run + kRescaleSlack;
      const float m_new = c_first ? mt : (need ? mt : m_run);
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      mu = m_new == -INFINITY ? 0.f : m_new;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) {  // product, two LDS reads, four vector instructions
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Phase B.
      {
        const u32x4_t pv = {pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
        for (int b = 0; b < DBLK; ++b) o[b] = mfma32(vf[1][b], pv, o[b]);
      }
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) kf[st] = *reinterpret_cast<const u32x4_t*>(kt_base + kofs[st]);
      exps(0, R_B);
#pragma unroll
      for (int i = 0; i < DBLK; ++i) {  // product, two LDS reads, six vector instructions
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Phase C (the second half of the K fragments is read while the first half is used).
      s_nxt = f32x16_t{};
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) s_nxt = mfma32(kf[st], qf[st], s_nxt);
      exps(R_B, 16);
      l_run = (c_first ? 0.f : l_run * alpha) + (lsum0 + lsum1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      // Keep the softmax results here: otherwise the compiler sinks them past the loop exit test
      // into the next iteration, where nothing overlaps them.
      asm volatile("" ::"v"(pk[0]), "v"(pk[1]), "v"(pk[2]), "v"(pk[3]), "v"(pk[4]), "v"(pk[5]), "v"(pk[6]),
                   "v"(pk[7]), "v"(l_run));

      // 6. Lazy rescale of the accumulator (tile j continues the item of tile j - 1).
      if (__any(need)) {
#pragma unroll
        for (int b = 0; b < DBLK; ++b) o[b] *= alpha;
      }
    }
    // 7. Tile j - 1 ended its item: normalise and store its rows (or split-key partials).  The
    // item's row range and slot were loaded at the end of the previous iteration (e_row0 ..).
    const int p_code = d_code[IP];
    if ((p_code & F_LAST) && !(p_code & F_IDLE) && code_it(p_code) < it_end) {
      const float l_tot = l_prev + other_half(l_prev);
      const int prow = e_row0 + tt;
      if (e_slot < 0) {
        // Normalised bf16 rows go through this wave's region of the Q buffer (free until the next
        // item's Q rows are loaded), so that each store writes whole 128-byte lines: written with
        // the Q layout (row n, unit u at u ^ swz_k(n)), read back the way the Q loads fill it, and
        // stored with the Q loads' offsets.
        // The additive sink appends exp(b) to the denominator: 2^(b log2(e) - m) in the units of
        // l (zero when b = -inf, which leaves the plain softmax bit for bit).
        const float inv = __builtin_amdgcn_rcpf(l_tot + fast_exp2(sink_log2 - m_prev));
        uint8_t* const stage = &qbuf[32 * RB * w];
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int j0 = 2 * t, j1 = 2 * t + 1;
            const uint32_t a0 = pack_bf16x2(o[b][4 * j0] * inv, o[b][4 * j0 + 1] * inv);
            const uint32_t a1 = pack_bf16x2(o[b][4 * j0 + 2] * inv, o[b][4 * j0 + 3] * inv);
            const uint32_t b0 = pack_bf16x2(o[b][4 * j1] * inv, o[b][4 * j1 + 1] * inv);
            const uint32_t b1 = pack_bf16x2(o[b][4 * j1 + 2] * inv, o[b][4 * j1 + 3] * inv);
            // Lane n holds d 16t + 4 half + {0..3} (a) and 16t + 8 + 4 half + {0..3} (b); after
            // swapping a of the upper half with b of the lower half, lane n holds d 16t + 0..7 and
            // lane n + 32 holds d 16t + 8..15 of block b: 16-byte unit 4b + 2t + half of row n.
            const auto r0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
            const auto r1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
            const int u = (32 * b + 16 * t + 8 * half) / 8;
            *reinterpret_cast<u32x4_t*>(stage + n * RB + 16 * (u ^ swz_k(n))) = u32x4_t{r0[0], r1[0], r0[1], r1[1]};
          }
        const rsrc_t ro = row_rsrc(O, e_row0, e_row_limit);  // rows past the item's last token are dropped
#pragma unroll
        for (int i = 0; i < DSTEPS; ++i) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + 1024 * i + 16 * lane);
          buf_store16_nt(v, ro, qdma[i]);  // whole lines, not read again by this kernel
        }
        since_q += DSTEPS;
        ex_prev += DSTEPS;
        if (lse && half == 0 && prow < e_row_limit)
          lse[int64_t(prow - q_row_base) * Hq + h] = (m_prev + __log2f(l_tot)) * kLn2;
      } else {
        const int64_t sl = int64_t(e_slot) * Hkv + g;
        int pl = lane;  // opaque: the address is formed here rather than held across the loop
        asm volatile("" : "+v"(pl));
        float* po = part_o + (sl * kRowsPerTile + w * 32 + (pl & 31)) * D + 4 * (pl >> 5);
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            *reinterpret_cast<f32x4_t*>(po + 32 * b + 8 * jj) =
                f32x4_t{o[b][4 * jj], o[b][4 * jj + 1], o[b][4 * jj + 2], o[b][4 * jj + 3]};
        since_q += 4 * DBLK;
        ex_prev += 4 * DBLK;
        if (half == 0) {
          part_ml[(sl * kRowsPerTile + rho) * 2] = m_prev;
          part_ml[(sl * kRowsPerTile + rho) * 2 + 1] = l_tot;
        }
      }
    }
    if ((p_code & F_LAST) && code_it(p_code) < it_end) {
#pragma unroll
      for (int b = 0; b < DBLK; ++b) o[b] = f32x16_t{};
    }
    // The Q buffer is free once the epilogue that followed the last Q read is done.  Past the
    // workgroup's last item nothing is loaded: a load of no rows still writes zeros into the
    // buffer, and the last item's epilogue stages its rows there without waiting for it.
    if (q_state == 2) {
      if (q_next < it_end) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // staged rows read back before the refill
        issue_q(q_next);
        since_q = 0;
        ex_prev += DSTEPS;
      }
      q_state = 0;
    } else if (q_state == 1) {
      q_state = 2;
    }
    // Tile j ends its item: fetch the item's row range and slot for the next iteration's epilogue.
    if ((c_code & F_LAST) && c_valid) {
      const int4 rr = *reinterpret_cast<const int4*>(&items[code_it(c_code)].row0);  // row0, row_limit, a_*
      e_row0 = rr.x;
      e_row_limit = rr.y;
      e_slot = items[code_it(c_code)].slot;
    }
    // 8. The window slot of tile j - 2 takes tile j + NS + 1.
    take(d_start[INEW], d_code[INEW], d_row0[INEW]);
  };

  // Iterations j = -1 .. n_total (P.V of the last tile runs in iteration n_total), unrolled by WIN
  // = 6 so that every ring slot (j mod 3), S^T register set (j mod 2) and window index is a
  // compile-time choice.
  for (int j = -1; j <= n_total; j += WIN) {
    iteration(std::integral_constant<int, 0>{});
    if (j + 1 > n_total) break;
    iteration(std::integral_constant<int, 1>{});
    if (j + 2 > n_total) break;
    iteration(std::integral_constant<int, 2>{});
    if (j + 3 > n_total) break;
    iteration(std::integral_constant<int, 3>{});
    if (j + 4 > n_total) break;
    iteration(std::integral_constant<int, 4>{});
    if (j + 5 > n_total) break;
    iteration(std::integral_constant<int, 5>{});
  }
  // Drain this wave's direct-to-LDS loads (zero-size ones past the end) before the workgroup exits.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(uint16_t* __restrict__ O, float* __restrict__ lse,
                                                         const MergeItem* __restrict__ merges,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, int Hq, int Hkv, int G,
                                                         int q_row_base, float sink_log2) {
  attn_merge_block<D, 32>(blockIdx.x, O, lse, merges, part_o, part_ml, Hq, Hkv, G, q_row_base, sink_log2);
}

template <int D, int G>
static hipError_t launch_attn_t(const AttnLaunch& a, hipStream_t stream) {
  if (a.n_items > 0) {
    const dim3 grid(unsigned(a.wg_per_head * a.num_kv_heads));
    if (a.ev_start) {
      hipError_t e = hipEventRecord(a.ev_start, stream);
      if (e != hipSuccess) return e;
    }
    if (a.rope == 0)
      attn_fwd_kernel<D, G, kFwdSlots, 0><<<grid, 256, 0, stream>>>(
          a.Q, a.K, a.V, a.O, a.lse, a.items, a.ranges, a.part_o, a.part_ml, a.num_q_heads, a.num_kv_heads,
          a.scale_log2, a.q_row_base, a.sink_log2, nullptr, nullptr);
    else if (a.rope == 1)
      attn_fwd_kernel<D, G, kFwdSlots, 1><<<grid, 256, 0, stream>>>(
          a.Q, a.K, a.V, a.O, a.lse, a.items, a.ranges, a.part_o, a.part_ml, a.num_q_heads, a.num_kv_heads,
          a.scale_log2, a.q_row_base, a.sink_log2, a.rope_cs, a.item_pidx);
    else
      attn_fwd_kernel<D, G, kFwdSlots, 2><<<grid, 256, 0, stream>>>(
          a.Q, a.K, a.V, a.O, a.lse, a.items, a.ranges, a.part_o, a.part_ml, a.num_q_heads, a.num_kv_heads,
          a.scale_log2, a.q_row_base, a.sink_log2, a.rope_cs, a.item_pidx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev_stop) {
      e = hipEventRecord(a.ev_stop, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (a.n_merges > 0 && !a.defer_merge) {
    const dim3 grid(unsigned(a.n_merges * a.num_kv_heads * merge_wg_per_tile<D>()));
    attn_merge_kernel<D><<<grid, 256, 0, stream>>>(a.O, a.lse, a.merges, a.part_o, a.part_ml, a.num_q_heads,
                                                   a.num_kv_heads, G, a.q_row_base, a.sink_log2);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (a.head_dim == 128) {
    switch (G) {
      case 1: return launch_attn_t<128, 1>(a, stream);
      case 2: return launch_attn_t<128, 2>(a, stream);
      case 4: return launch_attn_t<128, 4>(a, stream);
      case 8: return launch_attn_t<128, 8>(a, stream);
    }
  } else if (a.head_dim == 64) {
    switch (G) {
      case 1: return launch_attn_t<64, 1>(a, stream);
      case 2: return launch_attn_t<64, 2>(a, stream);
      case 4: return launch_attn_t<64, 4>(a, stream);
      case 8: return launch_attn_t<64, 8>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace br
