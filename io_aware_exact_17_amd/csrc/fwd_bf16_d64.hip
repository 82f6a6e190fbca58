// fwd_bf16_d64.hip — tiled exact-attention forward pass, bf16 in / bf16 out,
// head dimension 64, for gfx950.  (Head dimension 128 runs the kernel in
// fwd_bf16.hip: at d=64 the softmax outweighs the matrix work per score, and
// two waves per SIMD in opposite phase hide it better than one wave that
// pipelines both.)
//
// Method (FlashAttention explainer, cztcode.com/2026/5368, §2-§3; Flash
// Attention wiki note, astro-wiki, "Online Softmax", "Tiling" and the
// FlashAttention-2 notes): a workgroup owns a tile of query rows and streams
// the key/value tiles past it (query tile outer, key tile inner).  Each query
// row keeps a running maximum m, a running sum l of exp(s - m) and an
// unnormalised output u; when m grows, l and u are rescaled by exp(m_old -
// m_new); the division u / l happens once, after the last key tile.  Score and
// probability tiles live only in registers.  Key tiles wholly above the
// causal diagonal are never loaded (explainer §6).
//
// Mapping to CDNA4:
//  * 8 waves x 32 query rows = 256 rows per workgroup, one workgroup per CU,
//    two waves per SIMD.  Both products run on the matrix cores as
//    v_mfma_f32_32x32x16_bf16.
//  * The score tile is formed transposed, S^T = K Q^T, so every lane holds
//    one query column: row max and row sum are in-lane reductions plus one
//    exchange between lane halves (v_permlane32_swap); no reduction crosses
//    waves.  The S^T accumulators, rounded to bf16, are directly the B operand
//    of O^T += V^T P^T, so P never leaves registers.
//  * Two wave groups in opposite phase.  Waves 0-3 (group A) handle each key
//    tile as  S = K Q^T -> softmax -> O += P V;  waves 4-7 (group B, one on
//    each SIMD next to a group-A wave) as  O += P V of the previous tile ->
//    S = K Q^T -> softmax.  After each barrier the two waves sharing a SIMD
//    therefore run their vector-ALU softmax while the other one feeds the
//    matrix core, instead of both waiting on the same unit.
//  * K and V tiles (128 keys) go from HBM straight into LDS
//    (global_load_lds_dwordx4, 1 KB per wave instruction, no staging
//    registers), both row-major with each row's 16-byte chunks permuted by a
//    function of the row index, so K operand reads and transposing V reads
//    are free of bank conflicts.  The V^T operand comes from the row-major V
//    tile through ds_read_b64_tr_b16, addressed so that each lane receives,
//    for its own output dim, the keys its P registers hold.  Four K and five
//    V buffers (group B reads the previous position's V): tiles are copied
//    two positions ahead and a barrier follows every second position.
//  * exp is 2^x on v_exp_f32 with log2(e) folded into the scale.  The
//    reference maximum is not recomputed per tile: P is formed against the
//    current reference and only when a tile's P sum exceeds 2^8 (so some P
//    could exceed 256 before rounding to bf16) is the exact row maximum
//    taken, the reference moved and the output accumulator rescaled.  That
//    happens on the first tile and rarely afterwards; the mathematics is
//    unchanged because the final division uses the same reference.
//  * Work items (head, query tile) are listed heaviest query tile first,
//    heads fastest.  Dense runs one workgroup per CU, each taking one item
//    per round of G as one stream (see the kernel); since workgroups are dealt
//    round-robin to the 8 XCDs, when G (the CU count, 256, once there are
//    that many items) and B*H are multiples of 8 every item of a head lands
//    on the same XCD and shares its K/V in that XCD's L2.
#include <atomic>

#include "cdna4.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr int kThreads = 512;
constexpr int kBR = 256;          // query rows per workgroup (8 waves x 32)
constexpr int kKBuf = 4;          // LDS K buffers
constexpr int kVBuf = 5;          // LDS V buffers (group B reads the previous position's V)
constexpr float kSumBound = 256.f;  // a tile's P sum per lane half stays <= 2^8
constexpr int kPrefetch = 6;      // LDS operand reads kept ahead of the matrix cores
constexpr int kMaxDevices = 64;   // devices whose CU count is cached

template <int D>
struct FwdCfg {
  static constexpr int BC = 8192 / D;    // keys per tile: 128 for d=64
  static constexpr int KS = D / 16;      // k-steps of S^T = K Q^T
  static constexpr int NKB = BC / 32;    // 32-key blocks per tile
  static constexpr int NDB = D / 32;     // 32-row blocks of O^T
  static constexpr int ROWB = D * 2;     // bytes per tile row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int TILE = BC * ROWB;            // bytes per K or V tile
  static constexpr int RPI = 1024 / ROWB;           // tile rows per 1 KB wave instruction
  static constexpr int IPW = TILE / 1024 / (kThreads / 64);  // wave instructions per tile per wave
  static constexpr int OST = 2048;  // per-wave O staging (16 rows)
  static constexpr int LDS_BYTES = (kKBuf + kVBuf) * TILE + 8 * OST;
  static_assert(D == 64, "the LDS layout below is written for d = 64");
  static_assert(IPW * 1024 * (kThreads / 64) == TILE, "tile copies split evenly over the waves");
};

// LDS slot of 16-byte chunk c of tile row r (rows of 128 bytes, two per
// 256-byte bank line): c ^ f(r) with f(r) = (bit 1 of r) << 2 | bits 2-3 of
// r.  A K operand read (one chunk of 16 consecutive rows per 16 lanes) and a
// transposing V read (4 rows x 4 chunks) then touch 16 distinct 16-byte bank
// groups.  The permutation is its own inverse.
__device__ __forceinline__ int swz64(int r, int c) {
  return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// The work is a list of items, one per (sequence or batch-head, query tile),
// heaviest query tile first and heads fastest.  Workgroup g takes one item
// per round of G (G = number of workgroups; odd rounds in reverse order of
// 8-workgroup blocks, which balances causal work) and walks them as one stream
// of positions, one per key tile of each item in turn (an item with no
// visible key still takes one position, for its epilogue).  The staging of
// tiles two positions ahead, the lag of wave group B and the fetch of the
// next item's Q all run across item boundaries, so a workgroup pays for the
// pipeline's fill and drain once, not once per query tile.
//
// VARLEN: a packed batch of sequences (token-major [T, H, d], sequence b owns
// query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1, LSE
// [H, total_q]); items run sequence by sequence (the longest sequence's query
// tiles x H per sequence), and items past a sequence's last query tile are
// empty and skipped.  Otherwise dense [B, H, N, d].
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int Nq_dense, int Nk_dense,
    float c, int negate_q, int n_qtiles, int n_items, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int H, int total_q) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  constexpr int ROWB = C::ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  lds_char* const lds = (lds_char*)smem;  // kKBuf K tiles, kVBuf V tiles, then 2 KB of O staging per wave
  constexpr int VREG = kKBuf * C::TILE;   // byte offset of the V tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool group_b = wave >= 4;
  const int col = lane & 31;   // query column of this lane in S^T / O^T
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group this lane holds
  const int G = (int)gridDim.x;
  const int rs = VARLEN ? H * D : D;  // elements between consecutive rows of a head

  // Non-causal dense launches whose rounds are whole and whose XCDs' slots
  // split into whole heads deal every query tile of a head to one XCD in one
  // round (the slots of an XCD are g mod 8 = x), so the head's K/V is fetched
  // from HBM once and shared through that XCD's L2 (B=64 H=16 N=1024: HBM
  // reads ~3x the compulsory Q+K+V before, +15% speed).  Causal launches keep
  // heaviest-first rounds: mixing a head's unequal query tiles in one round
  // measured 5-33% slower, depending on the order of the tiles.
  const bool grouped =
      !VARLEN && !CAUSAL && (G & 7) == 0 && ((G >> 3) % n_qtiles) == 0 && n_items % G == 0;

  // ------------------------------------------------------------- the items
  // An item is kept as a few integers; row bases, lengths and tile counts
  // are derived on use (dense: from the kernel arguments), so the three
  // cursors below cost few scalar registers.
  struct Item {
    int qt;      // query tile
    int bh;      // batch-head (dense) or head (varlen)
    int qs, ks;  // varlen: the sequence's first query and key rows
    int nq, nk;  // varlen: the sequence's query and key counts
  };
  auto Nq_of = [&](const Item& it) -> int {
    if constexpr (VARLEN) return it.nq;
    else return Nq_dense;
  };
  auto Nk_of = [&](const Item& it) -> int {
    if constexpr (VARLEN) return it.nk;
    else return Nk_dense;
  };
  auto q0_of = [&](const Item& it) -> int { return it.qt * kBR; };
  auto qbase_of = [&](const Item& it) -> size_t {  // elements
    if constexpr (VARLEN) return ((size_t)it.qs * H + it.bh) * D;
    else return (size_t)it.bh * Nq_dense * D;
  };
  auto kbase_of = [&](const Item& it) -> size_t {
    if constexpr (VARLEN) return ((size_t)it.ks * H + it.bh) * D;
    else return (size_t)it.bh * Nk_dense * D;
  };
  auto lse_base_of = [&](const Item& it) -> size_t {
    if constexpr (VARLEN) return (size_t)it.bh * total_q + it.qs;
    else return (size_t)it.bh * Nq_dense;
  };
  // Key tiles of the item (causal: up to the diagonal of its last row).
  auto n_tiles_of = [&](const Item& it) -> int {
    const int Nk = Nk_of(it);
    const int kv_end = CAUSAL ? min(Nk, q0_of(it) + kBR + Nk - Nq_of(it)) : Nk;
    return kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  };
  // Returns false for an empty item (a query tile past its sequence's end).
  auto item_info = [&](int i, Item& it) -> bool {
    if constexpr (VARLEN) {
      const int per = n_qtiles * H;
      const int b = i / per, r = i - b * per;
      it.bh = r % H;
      it.qt = n_qtiles - 1 - r / H;
      it.qs = cu_q[b];
      it.ks = cu_k[b];
      it.nq = cu_q[b + 1] - it.qs;
      it.nk = cu_k[b + 1] - it.ks;
      return it.qt * kBR < it.nq;
    } else {
      if (grouped) {
        // round r, slot gg of the round (gg mod 8 = the workgroup's XCD): the
        // G/8 slots of an XCD take the n_qtiles query tiles of G/8/n_qtiles
        // heads
        const int r = i / G, gg = i - r * G;
        const int x = gg & 7, k = gg >> 3;
        it.qt = k % n_qtiles;
        it.bh = r * (G / n_qtiles) + x * (G / 8 / n_qtiles) + k / n_qtiles;
      } else {
        it.qt = n_qtiles - 1 - i / BH;
        it.bh = i % BH;
      }
      return true;
    }
  };
  // Key tiles this wave's 32 rows need (causal: up to its last row's diagonal).
  auto tiles_of_wave = [&](const Item& it) -> int {
    const int Nk = Nk_of(it);
    const int end = CAUSAL ? min(Nk, q0_of(it) + wave * 32 + 32 + Nk - Nq_of(it)) : Nk;
    return end > 0 ? (end + BC - 1) / BC : 0;
  };
  // Round r of the stream gives workgroup g item r*G + g on even rounds;
  // odd rounds run the round backwards in blocks of 8 workgroups (item
  // r*G + G-8 - (g & ~7) + (g & 7)), so g mod 8, and with it the XCD that
  // holds a head's K/V, stays the same (plain G-1-g when G is not a multiple
  // of 8).  Items are numbered heaviest first, so the reversed direction
  // pairs a round's heavy items with the next round's light ones: with fewer
  // items per query-tile level than workgroups (one long causal sequence
  // over few heads), a plain stride would hand the low workgroups the
  // heaviest item of every round.  Past the end: n_items.
  const int g_rev = (G & 7) == 0 ? G - 8 - ((int)blockIdx.x & ~7) + ((int)blockIdx.x & 7)
                                 : G - 1 - (int)blockIdx.x;
  auto slot = [&](int r) -> int {
    const long long i = (long long)r * G + ((r & 1) ? g_rev : (int)blockIdx.x);
    return i < n_items ? (int)i : n_items;
  };
  // A stream position: key tile j of this workgroup's item `item` (round
  // r), which spans n_pos = max(n_tiles, 1) positions.  item >= n_items ends
  // the stream.
  struct Cursor {
    int r, item, j, n_pos;
    Item it;  // the item's description (valid while item < n_items)
  };
  auto settle = [&](Cursor& cu) {  // move to the first non-empty item at or after round cu.r
    while (cu.item < n_items && !item_info(cu.item, cu.it)) cu.item = slot(++cu.r);
    cu.j = 0;
    cu.n_pos = cu.item < n_items ? max(n_tiles_of(cu.it), 1) : 0;
  };
  auto advance = [&](Cursor& cu) {
    if (++cu.j < cu.n_pos) return;
    cu.item = slot(++cu.r);
    settle(cu);
  };

  Cursor cur;
  cur.r = 0;
  cur.item = slot(0);
  settle(cur);
  if (cur.item >= n_items) return;  // uniform: no work for this workgroup

  // Q^T operand: lane holds Q[qi][16s + 8*half + 0..7].  Rows past Nq read
  // row Nq-1 (their results are never stored).
  const uint32_t flip = negate_q ? 0x80008000u : 0u;  // exact sign flip for a negative scale
  auto load_q = [&](const Item& it, u32x4 (&dst)[C::KS]) {
    const int qi = q0_of(it) + wave * 32 + col;
    const u32x4* src =
        reinterpret_cast<const u32x4*>(Q + qbase_of(it) + (size_t)min(qi, Nq_of(it) - 1) * rs);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) dst[s] = src[2 * s + half];
  };
  bf16x8 qf[C::KS];
  u32x4 qn[C::KS];  // the next item's Q, fetched one position ahead
  auto take_q = [&]() {
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qn[s] ^ flip);
  };
  load_q(cur.it, qn);
  take_q();
  // At the last position of an item, fetch the next item's Q into qn.
  auto prefetch_q = [&](const Cursor& cu) {
    if (cu.j != cu.n_pos - 1) return;
    Cursor nx;
    nx.r = cu.r + 1;
    nx.item = slot(nx.r);
    settle(nx);
    if (nx.item < n_items) load_q(nx.it, qn);
  };

  // ---------------------------------------------------------- tile staging
  // K and V tiles (BC keys x 128 bytes, row-major, 16-byte chunks permuted
  // by swz64) go from memory straight into LDS with global_load_lds_dwordx4:
  // wave instruction ii fills tile rows ii*RPI .. ii*RPI+RPI-1 (1 KB, lane
  // l at byte 16 l, i.e. row l / CPR, slot l % CPR), so the lane fetches the
  // chunk that slot holds.  Each of the 8 waves issues IPW instructions per
  // operand.  Keys past Nk fetch row Nk-1 (finite values whose scores are
  // masked to -inf).  Stream position p uses K buffer p % kKBuf and V buffer
  // p % kVBuf; a position with no key tile (an item with no visible key)
  // copies nothing.
  const int ld_row = lane / C::CPR;
  const int ld_slot = lane % C::CPR;
  const uint32_t rsb = (uint32_t)rs * 2;  // bytes between consecutive rows of a head
  const uint32_t lds_wave =
      (uint32_t)(size_t)lds + __builtin_amdgcn_readfirstlane(wave) * C::IPW * 1024;  // uniform
  auto issue_tile = [&](const Cursor& cu, int p) {
    const Item& it = cu.it;
    if (n_tiles_of(it) == 0) return;
    const int k0 = cu.j * BC;
    const int last = Nk_of(it) - 1 - k0;
    const char* kg = reinterpret_cast<const char*>(K + kbase_of(it) + (size_t)k0 * rs);
    const char* vg = reinterpret_cast<const char*>(V + kbase_of(it) + (size_t)k0 * rs);
    uint32_t kdst = lds_wave + (p % kKBuf) * C::TILE;
    uint32_t vdst = lds_wave + VREG + (p % kVBuf) * C::TILE;
    asm volatile("" : "+s"(kdst), "+s"(vdst));
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) {
      const int r = (wave * C::IPW + i) * C::RPI + ld_row;
      const uint32_t off = (uint32_t)min(r, last) * rsb + (uint32_t)(swz64(r, ld_slot) * 16);
      copy_to_lds(kg, off, kdst + i * 1024);
      copy_to_lds(vg, off, vdst + i * 1024);
    }
  };

  // LDS read offsets.  K operand of k-step s: key row col (+32 per key
  // block), chunk 2s + half.  V^T operand of dim block db for a 16-key group
  // (two transposing reads cc = 0, 1): lane l addresses key 8cc + 4 half +
  // (l%16)/4 of the group and dims d..d+3, d = 32 db + 16 ((l/16)%2) +
  // 4 (l%4); ds_read_b64_tr_b16 then hands each lane, for its own dim, the
  // four keys its P registers hold (keys 4h..4h+3 and 8+4h..8+4h+3 of the
  // group for lane half h).  The permutation depends on the row modulo 16,
  // so key blocks and groups are immediate offsets.
  uint32_t k_off[C::KS];
#pragma unroll
  for (int st = 0; st < C::KS; ++st) k_off[st] = (uint32_t)(col * ROWB + swz64(col, 2 * st + half) * 16);
  uint32_t v_off[2][C::NDB];
  {
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int key = 8 * cc + 4 * half + ((lane & 15) >> 2);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d = 32 * db + tr_dim;
        v_off[cc][db] = (uint32_t)(VREG + key * ROWB + swz64(key, d >> 3) * 16 + (d & 7) * 2);
      }
    }
  }

  // ------------------------------------------------------ per-tile stages
  f32x16 oacc[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) oacc[i] = f32x16{};
  float m_ref = kNegInf;  // reference maximum, log2 units (score * c)
  float l_part = 0.f;     // this lane half's share of the row sum
  f32x16 sacc[C::NKB];
  uint32_t pk[C::NKB][8];  // bf16 P pairs of the latest softmax

  // Matrix-core loops keep the LDS operands of kPrefetch products in
  // flight (R reads per product): the schedule is pinned to kPrefetch * R
  // reads, then (1 MFMA, R reads) groups, then the remaining MFMAs, so no
  // MFMA waits on a read issued just before.
  auto pipeline_schedule = [&](auto n_mfma, auto reads_per_mfma) {
    constexpr int N = decltype(n_mfma)::value;
    constexpr int R = decltype(reads_per_mfma)::value;
#pragma unroll
    for (int i = 0; i < kPrefetch * R; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kPrefetch < N) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    }
  };

  // The wave feeding the matrix core runs at raised issue priority, so the
  // neighbouring wave's vector work fills the gaps instead of delaying it.
  auto qk = [&](int p) {
    __builtin_amdgcn_s_setprio(1);
    const lds_char* sk = lds + (p % kKBuf) * C::TILE;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < C::KS; ++st)
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const lds_bf16x8*>(sk + kb * 32 * ROWB + k_off[st]);
        sacc[kb] = mfma_32x32x16(a, qf[st], sacc[kb]);
      }
    pipeline_schedule(std::integral_constant<int, C::KS * C::NKB>{}, std::integral_constant<int, 1>{});
    __builtin_amdgcn_s_setprio(0);
  };

  auto pv = [&](int p) {
    __builtin_amdgcn_s_setprio(1);
    // This lane's read addresses in the buffer, formed once per call and
    // hidden from re-association, so the 16-key group offsets below fold
    // into the reads' immediate offsets instead of costing an add per read.
    uint32_t vb[2][C::NDB];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        vb[cc][db] = (uint32_t)(size_t)lds + (p % kVBuf) * C::TILE + v_off[cc][db];
        asm volatile("" : "+v"(vb[cc][db]));
      }
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 b = __builtin_bit_cast(
            bf16x8, u32x4{pk[kb][4 * t], pk[kb][4 * t + 1], pk[kb][4 * t + 2], pk[kb][4 * t + 3]});
        constexpr int kGrpBytes = 16 * ROWB;  // one 16-key group
        const int g = 2 * kb + t;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const u32x2 lo = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)(vb[0][db] + g * kGrpBytes)));
          const u32x2 hi = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)(vb[1][db] + g * kGrpBytes)));
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          oacc[db] = mfma_32x32x16(a, b, oacc[db]);
        }
      }
    pipeline_schedule(std::integral_constant<int, C::NKB * 2 * C::NDB>{}, std::integral_constant<int, 2>{});
    __builtin_amdgcn_s_setprio(0);
  };

  // Masks keys past the end and, on diagonal tiles, keys after the query;
  // then P = 2^(s*c - m) against the current reference m, the row sum and
  // the bf16 pairs of P.  The reference only has to keep every P small, so
  // instead of a row maximum per tile the tile's own sum decides: if any
  // lane's share exceeds 2^tau, or some row has no reference yet, the wave
  // takes the exact path — row maximum, new reference, O and l rescaled, P
  // formed from the new reference.  Either way every P <= 2^tau.
  auto exp_tile = [&](float m_use, float& lsum) {
    lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_hw(__builtin_fmaf(sacc[kb][r], c, -m_use));
        const float p1 = exp2_hw(__builtin_fmaf(sacc[kb][r + 1], c, -m_use));
        lsum += p0 + p1;
        pk[kb][r >> 1] = pack_bf16x2(p0, p1);
      }
  };
  auto softmax = [&](const Item& it, int j) {
    const int k0 = j * BC;
    const int Nk = Nk_of(it);
    const int off = Nk - Nq_of(it);  // bottom-right causal alignment
    const int wq0 = q0_of(it) + wave * 32;
    const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > wq0 + off);
    if (__builtin_expect(need_mask, 0)) {
      [[unlikely]];
      // Register r of block kb holds key k0 + 32 kb + 4 half + 8 (r/4) + r%4;
      // it is hidden iff 8 (r/4) + r%4 > room(kb).  Each test and its select
      // go through VCC as one pair, so the 64 tests never sit in scalar
      // registers at once.
      // The compiler does not guard inline assembly against reading a
      // matrix product too early: 32 wait states first (more than an
      // 8-pass product needs before a vector read of its result).
      const int lim = CAUSAL ? min(Nk - 1, wq0 + col + off) : Nk - 1;
      const float ninf = kNegInf;
      asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        const int room = lim - k0 - kb * 32 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          asm volatile("v_cmp_gt_i32 vcc, %[pos], %[room]\n\tv_cndmask_b32 %[x], %[x], %[ninf], vcc"
                       : [x] "+v"(sacc[kb][r])
                       : [pos] "i"(8 * (r >> 2) + (r & 3)), [room] "v"(room), [ninf] "v"(ninf)
                       : "vcc");
      }
    }
    // Until a row has a reference (m_ref = -inf: its first tile with a
    // visible key) the wave goes straight to the exact path; otherwise it
    // takes the exact path only when the tile's sum bound fails.
    float lsum = 0.f;
    bool exact = wave_any(m_ref == kNegInf);
    if (__builtin_expect(!exact, 1)) {
      exp_tile(m_ref, lsum);
      exact = wave_any(!(lsum <= kSumBound));
    }
    if (__builtin_expect(exact, 0)) {
      [[unlikely]];
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_across_halves(mx);
      const float m_new = fmaxf(m_ref, mx * c);  // c > 0, so -inf stays -inf
      // Rows without a reference have O = 0 and l = 0 (no P was formed
      // against m = -inf), so a wave where no row had one skips the rescale.
      if (wave_any(m_ref != kNegInf && m_new != m_ref)) {
        const float alpha = m_new != m_ref ? exp2_hw(m_ref - m_new) : 1.f;  // 0 from -inf
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < C::NDB; ++i) oacc[i] *= alpha;
      }
      m_ref = m_new;
      exp_tile(m_ref == kNegInf ? 0.f : m_ref, lsum);
    }
    l_part += lsum;
  };

  // One division per row, O in bf16, LSE = ln2 * (m + log2 l); then the
  // running state starts again for the next item.
  auto epilogue = [&](const Item& it) {
    const int qi = q0_of(it) + wave * 32 + col;
    const float l_tot = sum_across_halves(l_part);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (half == 0 && qi < Nq_of(it))
      LSE[lse_base_of(it) + qi] = l_tot > 0.f ? (m_ref + log2_hw(l_tot)) * kLn2 : kNegInf;
    // O leaves through this wave's 2 KB of LDS, 16 rows at a time: rows
    // written with their 16-byte chunks at slots c ^ (row % 8), read back
    // as whole rows and stored with 16-byte non-temporal writes (8 rows per
    // instruction; O is not read again, so its lines need not stay in L2).
    // Same wave: program order orders the reads after the writes, and the
    // second half's writes after the first half's reads.
    lds_char* const ost = lds + (kKBuf + kVBuf) * C::TILE + wave * C::OST;
    const int row0 = q0_of(it) + wave * 32;
    bf16* const obase = O + qbase_of(it);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      if ((col >> 4) == h2) {
        const int rr = col & 15;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                             pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
            const int chunk = 4 * db + g;  // dims 8 chunk .. +7; this lane half holds +4 half .. +3
            *reinterpret_cast<lds_u32x2*>(ost + rr * 128 + ((chunk ^ (rr & 7)) * 16) + 8 * half) = w;
          }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ci = 64 * i + lane;
        const int rr = ci >> 3, cc = ci & 7;
        const u32x4 w = *reinterpret_cast<const lds_u32x4*>(ost + rr * 128 + ((cc ^ (rr & 7)) * 16));
        const int row = row0 + 16 * h2 + rr;
        if (row < Nq_of(it)) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(obase + (size_t)row * rs + cc * 8));
      }
    }
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) oacc[i] = f32x16{};
    m_ref = kNegInf;
    l_part = 0.f;
  };

  // ------------------------------------------------------------- main loop
  // The copies of position p+2 are issued at the start of position p, and
  // every second position (p odd) ends with a wait for all copies and a
  // barrier.  Position p's copies go to K buffer (p+2) % 4, last read at
  // position p-2, and V buffer (p+2) % 5, last read at p-2 by group B; a
  // barrier lies between (after p-1 when p is even, after p-2 when it is
  // odd).  Position p reads what was copied at p-2 and waited for at that
  // same barrier.  Positions 0 and 1 are copied before the first barrier;
  // `ld` is the next position to copy.
  Cursor ld = cur;
  issue_tile(ld, 0);
  advance(ld);
  if (ld.item < n_items) {
    issue_tile(ld, 1);
    advance(ld);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // Group B finishes the previous position's P V first, so the stream ends
  // with one extra step in which only group B works.
  Cursor prv;  // the position before cur (none yet)
  prv.item = n_items;
  for (int p = 0; cur.item < n_items || prv.item < n_items; ++p) {
    const bool have_cur = cur.item < n_items;
    const Item& ic = cur.it;
    paranoid_sync();
    if (ld.item < n_items) {
      issue_tile(ld, p + 2);
      advance(ld);
    }
    paranoid_sync();
    if (!group_b) {
      if (have_cur) {
        prefetch_q(cur);
        if (cur.j < tiles_of_wave(ic)) {
          qk(p);
          softmax(ic, cur.j);
          pv(p);
        }
        if (cur.j == cur.n_pos - 1) {
          epilogue(ic);
          take_q();
        }
      }
    } else {
      if (prv.item < n_items) {
        const Item& ip = prv.it;
        if (prv.j < tiles_of_wave(ip)) pv(p - 1);
        if (prv.j == prv.n_pos - 1) {
          epilogue(ip);
          if (have_cur) take_q();
        }
      }
      if (have_cur) {
        prefetch_q(cur);
        if (cur.j < tiles_of_wave(ic)) {
          qk(p);
          softmax(ic, cur.j);
        }
      }
    }
    if (p & 1) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
    }
    prv = cur;
    if (have_cur) advance(cur);
  }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs& a) {
  const int n_qtiles = (int)(((long long)a.Nq + kBR - 1) / kBR);
  const int BH = a.B * a.H;
  // c > 0 keeps masked scores (-inf) at -inf after scaling.  A zero scale
  // becomes 1e-30: every product with a finite score then rounds away
  // against the reference, so the weights are exactly uniform, as for 0.
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  const int neg = a.scale < 0.f ? 1 : 0;
  const int n_items = n_qtiles * BH;
  // Dense: one workgroup per CU (the LDS and registers of one workgroup fill
  // a CU), each walking every G-th item; the items alternate over the heads,
  // so with B*H a multiple of 8 a head's items stay on one XCD.  Varlen: one
  // workgroup per item, so the hardware balances sequences of any length.
  int G = n_items;
  if constexpr (!VARLEN) {
    int cus = 0;
    const hipError_t e = cu_count(a.stream, &cus);
    if (e != hipSuccess) return e;
    G = min(n_items, cus);
  }
  const dim3 grid((unsigned)G);
  const dim3 block(kThreads);
  void* args[] = {(void*)&a.q,    (void*)&a.k,   (void*)&a.v,        (void*)&a.o,
                  (void*)&a.lse,  (void*)&BH,    (void*)&a.Nq,       (void*)&a.Nk,
                  (void*)&c,      (void*)&neg,   (void*)&n_qtiles,   (void*)&n_items,
                  (void*)&a.cu_q, (void*)&a.cu_k, (void*)&a.H,       (void*)&a.total_q};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, CAUSAL, VARLEN>), grid,
                         block, args, 0, a.stream);
}

}  // namespace

// Compute units of the device `stream` belongs to (the null stream: the
// current device), read once per device and kept: a device property, not
// state that changes between calls.
hipError_t cu_count(hipStream_t stream, int* cus) {
  static std::atomic<int> cache[kMaxDevices];
  hipDevice_t dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidDevice;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return hipSuccess;
}

hipError_t launch_fwd_bf16_d64(const FwdArgs& a) {
  if (a.cu_q) return a.causal ? launch<64, true, true>(a) : launch<64, false, true>(a);
  return a.causal ? launch<64, true, false>(a) : launch<64, false, false>(a);
}

}  // namespace fa
