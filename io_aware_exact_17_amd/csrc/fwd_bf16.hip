// fwd_bf16.hip — tiled exact-attention forward pass, bf16 in / bf16 out, for
// gfx950.
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
// Mapping to CDNA4 (head dimension 128; d = 64 runs fwd_bf16_d64.hip):
//  * 4 waves x 64 query rows = 256 rows per workgroup, one workgroup (one wave
//    per SIMD) per CU.  A wave holds its rows as two 32-row blocks and both
//    products run on the matrix cores as v_mfma_f32_32x32x16_bf16; every K or
//    V operand read from LDS feeds both row blocks, which halves the LDS read
//    traffic per matrix instruction against 32-row waves.  O^T lives in the
//    accumulation registers, and so does Q.
//  * The score block is formed transposed, S^T = K Q^T, so every lane holds
//    one query column: row max and row sum are in-lane reductions plus one
//    exchange between lane halves (v_permlane32_swap); no reduction crosses
//    waves.  The S^T products are single-instruction inline assembly so the
//    scores land in vector registers, where the softmax reads them.  Rounded
//    to bf16 they are directly the B operand of O^T += V^T P^T, so P never
//    leaves registers.
//  * K and V tiles (64 keys) go from HBM straight into LDS
//    (global_load_lds_dwordx4, 1 KB per wave instruction, no staging
//    registers), both row-major, with the 16-byte chunks of each row permuted
//    by an XOR of a function of the row index so that both kinds of operand
//    read below touch 16 distinct 16-byte bank groups per 256 bytes.  The V^T
//    operand comes from the row-major V tile through the transposing LDS read
//    ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
//    element i%4 of the 8-byte pieces addressed by lanes i0 + (i%16)/4 + 4k,
//    k = 0..3, so addresses are chosen such that a lane receives, for its own
//    output dim, the four keys its P registers hold.  Four LDS buffers per
//    operand; K tiles are requested four tiles ahead, V tiles three, and
//    waited for explicitly; one barrier per 64 keys.
//  * Software pipeline over 32-key blocks inside each wave: while the scores
//    of block b go through the softmax on the vector ALUs, the matrix cores
//    compute the scores of block b+1 and add block b-1's P V into O.  A step
//    is four quarters, each with four S^T and four P V instructions, eight
//    scores of softmax and the LDS reads for the next quarter issued first.
//  * exp is 2^x on v_exp_f32 with log2(e) folded into the scale.  P is formed
//    against the current reference maximum; only when a block's P sum per
//    lane exceeds 2^8 (so some P could exceed 256 before rounding to bf16) is
//    the exact row maximum taken, the reference moved and O and l rescaled.
//    The mathematics is unchanged: the final division uses the same
//    reference.  Masks (causal diagonal, keys past the end) act on P, so they
//    are exact whatever the sign of the scale.
//  * Work items (head, query tile) are listed heaviest query tile first,
//    heads fastest.  Dense: one workgroup per CU, each taking one item per
//    round of G (the CU count) as one stream of tile positions: the K/V
//    copies run ahead across item boundaries, the next item's Q is requested
//    at the end of the item before, and O leaves through the LDS freed by
//    the last V tile, so the pipeline fills once per workgroup, not once per
//    query tile.  Odd rounds go in reverse order of 8-workgroup blocks, which
//    pairs heavy and light causal tiles on every CU.  Workgroups are dealt
//    round-robin to the 8 XCDs, so with G and B*H multiples of 8 every item
//    of a head lands on the same XCD and shares its K/V in that XCD's L2.
//    Varlen and block-sparse launch one workgroup per item, which the
//    hardware balances over sequences of any length or sparsity.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBR = 256;             // query rows per workgroup (4 waves x 64)
constexpr int kBC = 64;              // keys per staged tile (two 32-key blocks)
constexpr int kNBuf = 4;             // LDS buffers per operand
constexpr float kSumBound = 256.f;   // a block's P sum per lane stays <= 2^8
constexpr int kMaxSparseTiles = 1024;  // key tiles a block-sparse walk may list (Nk <= 65536)

template <int D>
struct FwdCfg {
  static constexpr int KS = D / 16;         // k-steps of S^T = K Q^T
  static constexpr int NDB = D / 32;        // 32-row blocks of O^T
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int TILE = kBC * D;      // elements per K or V tile
  static constexpr int RPI = 64 / CPR;      // tile rows per 1 KB wave instruction
  static constexpr int IPT = kBC / RPI;     // wave instructions per tile
  static constexpr int IPW = IPT / kWaves;  // ... per wave
  static_assert(IPW * kWaves == IPT, "tile loads split evenly over the waves");
};

// LDS slot of 16-byte chunk c of tile row r: c ^ f(r).  With 256-byte bank
// lines, f maps the 16 rows of an aligned group to distinct values (K reads:
// 16 lanes, one chunk of 16 rows) and gives the 4 rows of an aligned group of
// four distinct high bits (transposing V reads: 4 rows x 4 chunks).
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {  // two 128-byte rows per bank line; bit 0 of r picks the half
    return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
}

// One k-step of S^T = K Q^T on the matrix core (v_mfma_f32_32x32x16_bf16)
// written as a single instruction, so that the scores land in vector
// registers, where the softmax reads them, while the Q operand stays in
// accumulation registers.  The compiler does not see these as matrix
// instructions, so the code orders them: a chain alternates its two row
// blocks (as compiled chains do), and the first vector-ALU read of a score
// comes three matrix instructions or a wait (products_done) after the last
// instruction of its chain.
__device__ __forceinline__ void qk_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void qk_next(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// Wait until at most the vector-memory operations a tile iteration issued
// are outstanding: its own K and V tile copies (IPW instructions each, if
// issued).  Operations complete in issue order, so everything older has
// then landed.
template <int IPW>
__device__ __forceinline__ void wait_vm(bool k, bool v) {
  const int kv = (k ? 1 : 0) + (v ? 1 : 0);
  if (kv == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW));
  else if (kv == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPW));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Scheduling pattern: N matrix instructions, each followed by its share of
// the transcendental (TRANS) and other vector (VALU) instructions; the
// first TRANS % N and VALU % N shares are one larger.
template <int N, int TRANS, int VALU, int I = 0>
__device__ __forceinline__ void mfma_valu_pattern() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr ((TRANS + N - 1 - I) / N > 0)
      __builtin_amdgcn_sched_group_barrier(0x400, (TRANS + N - 1 - I) / N, 0);
    if constexpr ((VALU + N - 1 - I) / N > 0)
      __builtin_amdgcn_sched_group_barrier(0x002, (VALU + N - 1 - I) / N, 0);
    mfma_valu_pattern<N, TRANS, VALU, I + 1>();
  }
}

// The rare paths replace the P pairs and row sums of the common path; they
// consume them first, so that the compiler cannot sink the common-path
// softmax out of the matrix-core quarters into the branch that keeps it.
__device__ __forceinline__ void consume(const uint32_t (&pk)[2][8], const float (&lsum)[2]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pk[rb][i]));
    asm volatile("" ::"v"(lsum[rb]));
  }
}

// 32 wait states: more than the matrix-instruction-to-vector-ALU distance
// an 8-pass product needs before its result may be read.  Used where a
// vector read of a product's result could follow it closely: after the
// first scores, before the rare rescale of O and before the epilogue.  In
// the steady state the fixed order of each quarter keeps at least three
// matrix instructions between the last product into a score register and
// its first read (next step), so no wait is needed there.
__device__ __forceinline__ void products_done() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15");
  __builtin_amdgcn_sched_barrier(0);
}

// Matrix-core operands of one quarter step, read from LDS one quarter ahead.
template <int D>
struct QuarterOps {
  bf16x8 k[D / 64];  // K operands of k-steps 2q', 2q'+1 (d=128) or q' (d=64)
  bf16x8 v[D / 64];  // V^T operands of dim blocks (q'%2)*NDB/2 + i
};

// VARLEN: a packed batch of sequences of different lengths, token-major
// ([T, H, d], rows of one head H*d elements apart), sequence b owning query
// rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1, LSE
// [H, total_q]; grid (the longest sequence's query tiles x H, B).
// Otherwise [B, H, N, d] with contiguous rows per head.
//
// SPARSE (dense layout only): key j is visible to query i only where the
// block mask [H, nqb, nkb] (64 x 64 blocks) admits the pair.  A wave's 64
// rows are one mask row; the workgroup walks the compacted list of key tiles
// any of its four mask rows admits, and a wave whose own row does not admit
// a listed tile masks all of it.
template <int D, bool CAUSAL, bool VARLEN, bool SPARSE>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int Nq_dense, int Nk_dense,
    float c, int n_qtiles, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    int H, int total_q, const uint8_t* __restrict__ bmask, int nqb, int nkb, int n_items) {
  using C = FwdCfg<D>;
  using Ops = QuarterOps<D>;
  constexpr int TB = C::TILE * 2;        // bytes per K or V tile
  constexpr int VREG = kNBuf * TB;       // byte offset of the V buffers
  constexpr int ROWB = D * 2;            // bytes per tile row
  constexpr int KQ = C::KS / 4;          // k-steps per quarter
  constexpr int VQ = C::NDB / 2;         // dim blocks per quarter
  // K buffers, V buffers and (streaming) 16 KB more, which with V buffer 3
  // stages O at an item's end.
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * kNBuf * C::TILE + (!VARLEN && !SPARSE ? C::TILE : 0)];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // query column of this lane in S^T / O^T
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group this lane holds

  // Work items.  Varlen and block-sparse: one item per workgroup, from the
  // grid.  Dense (STREAM): item it is query tile n_qtiles-1-it/BH of
  // (batch, head) it%BH -- heaviest first, heads fastest -- and workgroup g
  // of G (one per CU) takes item rG+g in round r, with odd rounds reversed
  // in blocks of 8 workgroups (rG+G-8-(g&~7)+(g&7): g mod 8, and so the XCD
  // that holds a head's K/V in its L2, is kept).  Its items form one stream
  // of 64-key tile positions; the K/V copies run ahead across item
  // boundaries and the next item's Q is requested at the end of the item
  // before, so the pipeline fills once per workgroup, not once per query
  // tile.
  constexpr bool STREAM = !VARLEN && !SPARSE;
  const int G = (int)gridDim.x;
  const int g = (int)blockIdx.x;
  auto item_at = [&](int r) -> long long {
    const int o = ((r & 1) && (G & 7) == 0) ? G - 8 - (g & ~7) + (g & 7) : g;
    return (long long)r * G + o;
  };
  auto valid_round = [&](int r) -> bool { return item_at(r) < n_items; };
  // Row strides in global memory (a head's rows are contiguous when dense).
  const size_t q_rs = VARLEN ? (size_t)H * D : (size_t)D;       // elements
  const uint32_t kv_rsb = VARLEN ? (uint32_t)(H * ROWB) : ROWB;  // bytes

  int qt = 0, Nq = Nq_dense, Nk = Nk_dense, head = 0;
  size_t qbase = 0, kbase = 0, lse_base = 0;  // elements
  // Key tiles an item's query tile reaches (dense).
  auto tiles_of_qt = [&](int t) -> int {
    const int kv_end = CAUSAL ? min(Nk, t * kBR + kBR + (Nk - Nq)) : Nk;
    return kv_end > 0 ? (kv_end + kBC - 1) / kBC : 0;
  };
  auto set_dense_item = [&](int it) {
    qt = n_qtiles - 1 - it / BH;
    const int bh = it % BH;
    head = bh % max(H, 1);
    qbase = (size_t)bh * Nq * D;
    kbase = (size_t)bh * Nk * D;
    lse_base = (size_t)bh * Nq;
  };
  if constexpr (VARLEN) {
    // One sequence after another (grid.y), so the workgroups running
    // together share that sequence's K/V in L2; within it, heaviest tile
    // first, heads fastest.
    const int h = (int)(blockIdx.x % H);
    const int b = (int)blockIdx.y;
    qt = n_qtiles - 1 - (int)(blockIdx.x / H);
    const int qs = cu_q[b], ks = cu_k[b];
    Nq = cu_q[b + 1] - qs;
    Nk = cu_k[b + 1] - ks;
    if (qt * kBR >= Nq) return;  // past this sequence's last query tile
    head = h;
    qbase = ((size_t)qs * H + h) * D;
    kbase = ((size_t)ks * H + h) * D;
    lse_base = (size_t)h * total_q + qs;
  } else if constexpr (SPARSE) {
    set_dense_item(g);
  } else {
    set_dense_item((int)item_at(0));
  }
  const int off = Nk - Nq;  // bottom-right causal alignment
  int q0, kv_end, n_cand, wq0, qi0, kv_end_w;
  auto set_rows = [&]() {
    q0 = qt * kBR;
    kv_end = CAUSAL ? min(Nk, q0 + kBR + off) : Nk;
    n_cand = kv_end > 0 ? (kv_end + kBC - 1) / kBC : 0;  // key tiles in causal reach
    wq0 = q0 + wave * 64;  // first query row of this wave
    qi0 = wq0 + col;       // this lane's row in row block 0 (+32 in block 1)
    kv_end_w = CAUSAL ? min(Nk, wq0 + 64 + off) : Nk;
  };
  set_rows();

  // Q^T operands: lane holds Q[row][16s + 8*half + 0..7] of both row blocks.
  // Rows past Nq read row Nq-1 (their results are never stored).  They live
  // in accumulation registers, where only the S^T products read them.
  bf16x8 qf[2][C::KS];
  auto load_q = [&](bf16x8 (&dst)[2][C::KS], size_t qb, int first_row) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const bf16* src = Q + qb + (size_t)min(first_row + col + 32 * rb, Nq - 1) * q_rs + 8 * half;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) dst[rb][s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
    }
  };
  load_q(qf, qbase, wq0);

  // Block-sparse: the list of key tiles (s_tile) that any of the four mask
  // rows of the workgroup admits, in order, with the admitting waves as bits
  // (s_vis); compacted with one ballot per wave and 256 candidates per pass.
  __shared__ uint16_t s_tile[SPARSE ? kMaxSparseTiles : 1];
  __shared__ uint8_t s_vis[SPARSE ? kMaxSparseTiles : 1];
  __shared__ int s_cnt[SPARSE ? kWaves : 1];
  int n_list = n_cand, nbw, njw;
  if constexpr (SPARSE) {
    const uint8_t* mrow = bmask + ((size_t)head * nqb + 4 * qt) * nkb;
    n_list = 0;
    for (int base = 0; base < n_cand; base += kThreads) {
      const int t = base + tid;
      unsigned vis = 0;
      if (t < n_cand) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (4 * qt + w < nqb && mrow[(size_t)w * nkb + t]) vis |= 1u << w;
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(vis != 0);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (lane == 0) s_cnt[wave] = __builtin_popcountll(bal);
      __syncthreads();
      int at = n_list;
      for (int w = 0; w < wave; ++w) at += s_cnt[w];
      if (vis) {
        s_tile[at + below] = (uint16_t)t;
        s_vis[at + below] = (uint8_t)vis;
      }
      n_list += s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
      __syncthreads();
    }
    // Listed tiles this wave's rows can reach causally (the list is sorted).
    const int lim_tile = kv_end_w > 0 ? (kv_end_w + kBC - 1) / kBC : 0;
    int cnt = 0;
    for (int i0 = 0; i0 < n_list; i0 += 64) {
      const int i = i0 + lane;
      const int ti = s_tile[min(i, kMaxSparseTiles - 1)];
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < n_list && ti < lim_tile));
    }
    njw = cnt;
    nbw = 2 * njw;
  }
  auto set_wave_blocks = [&]() {
    nbw = kv_end_w > 0 ? (kv_end_w + 31) / 32 : 0;  // 32-key blocks this wave needs
    njw = (nbw + 1) / 2;                             // tiles this wave needs
  };
  if constexpr (!SPARSE) set_wave_blocks();
  int n_tiles = n_list;
  int n_pos = STREAM ? (n_tiles + kNBuf - 1) / kNBuf * kNBuf : n_tiles;  // positions of the item
  // Key tile of list entry j (the identity when dense).  The walk also
  // forms the scores of the block after the last one; past the list that is
  // a tile beyond Nk, masked whole as in the dense walk.
  auto tile_of = [&](int j) -> int {
    if constexpr (SPARSE)
      return j < n_tiles ? __builtin_amdgcn_readfirstlane((int)s_tile[j]) : (Nk + kBC - 1) / kBC;
    else
      return j;
  };
  // First key of 32-key block b of the walk.
  auto key_pos = [&](int b) -> int {
    if constexpr (SPARSE) return tile_of(b >> 1) * kBC + 32 * (b & 1);
    else return 32 * b;
  };
  auto admitted = [&](int b) -> bool {
    if constexpr (SPARSE)
      return (b >> 1) < n_tiles && ((__builtin_amdgcn_readfirstlane((int)s_vis[b >> 1]) >> wave) & 1);
    else
      return true;
  };

  // ---------------------------------------------------------- tile staging
  // Wave w issues wave instructions w*IPW .. w*IPW+IPW-1 of a tile; wave
  // instruction ii fills tile rows ii*RPI .. ii*RPI+RPI-1 (1 KB, lane l at
  // byte 16 l), so lane l owns slot l%CPR of row ii*RPI + l/CPR and fetches
  // the chunk that slot holds.  Full tiles use a uniform tile address plus a
  // fixed lane offset; in a tile that crosses Nk, rows past Nk fetch row
  // Nk-1 (finite values whose P is masked to 0).
  const int ld_row = lane / C::CPR;
  const int ld_slot = lane % C::CPR;
  uint32_t g_off[C::IPW];
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    const int r = (wave * C::IPW + i) * C::RPI + ld_row;
    g_off[i] = (uint32_t)(r * kv_rsb + swz<D>(r, ld_slot) * 16);  // the permutation is its own inverse
  }
  const uint32_t lds_wave = (uint32_t)(size_t)lds + wave * C::IPW * 1024;
  auto issue = [&](const char* base, int region, int j) {
    const int tj = tile_of(j);
    const char* t = base + (size_t)tj * kBC * kv_rsb;
    uint32_t dst = lds_wave;
    asm volatile("" : "+s"(dst));
    dst += region;
    if ((tj + 1) * kBC <= Nk) {
#pragma unroll
      for (int i = 0; i < C::IPW; ++i) copy_to_lds(t, g_off[i], dst + i * 1024);
    } else {
      const int last = Nk - 1 - tj * kBC;
#pragma unroll
      for (int i = 0; i < C::IPW; ++i) {
        const int r = (wave * C::IPW + i) * C::RPI + ld_row;
        copy_to_lds(t, (uint32_t)(min(r, last) * kv_rsb + swz<D>(r, ld_slot) * 16), dst + i * 1024);
      }
    }
  };
  // The tile stream.  Copy position p (counted from the current item's
  // first position) is the current item's tile p while p < n_pos, else
  // tile p - n_pos of the next item that has key tiles (nx_bh >= 0: its
  // batch x head, nx_tiles its key tiles).  Items take a multiple of kNBuf
  // positions when streaming, so every item starts at buffer 0; positions
  // past an item's last tile copy nothing.  Position p goes to buffer
  // p % kNBuf.
  int nx_bh = -1, nx_tiles = 0;
  auto find_next = [&](int r) {  // the first item with key tiles from round r on
    nx_bh = -1;
    nx_tiles = 0;
    if constexpr (STREAM) {
      for (; valid_round(r); ++r) {
        const int it = (int)item_at(r);
        const int nt = tiles_of_qt(n_qtiles - 1 - it / BH);
        if (nt > 0) {
          nx_bh = it % BH;
          nx_tiles = nt;
          return;
        }
      }
    }
  };
  auto issue_pos = [&](const bf16* base, int region, int p) -> bool {
    if (p < n_pos) {
      if (p >= n_tiles) return false;
      issue(reinterpret_cast<const char*>(base + kbase), region, p);
      return true;
    }
    if constexpr (STREAM) {
      p -= n_pos;
      if (nx_bh < 0 || p >= nx_tiles) return false;
      issue(reinterpret_cast<const char*>(base + (size_t)nx_bh * Nk * D), region, p);
      return true;
    }
    return false;
  };
  auto issue_k = [&](auto buf, int p) -> bool { return issue_pos(K, decltype(buf)::value * TB, p); };
  auto issue_v = [&](auto buf, int p) -> bool { return issue_pos(V, VREG + decltype(buf)::value * TB, p); };

  // LDS read offsets for buffer 0, first 32-key half of the tile; the
  // buffer, the half and (for V) the 16-key group are immediate offsets,
  // since the row permutation depends on the row index modulo 16 only.
  //   K operand of k-step s: key row col, chunk 2s + half.
  //   V^T operand (transposing read cc of dim block db): lane l addresses key
  //   8cc + 4*half + (l%16)/4 and dims d..d+3, d = 32db + 16*((l/16)%2) + 4*(l%4).
  uint32_t k_off[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) k_off[s] = (uint32_t)(col * ROWB + swz<D>(col, 2 * s + half) * 16);
  uint32_t v_off[2][C::NDB];
  {
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int key = 8 * cc + 4 * half + ((lane & 15) >> 2);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d = 32 * db + tr_dim;
        v_off[cc][db] = (uint32_t)(VREG + key * ROWB + swz<D>(key, d >> 3) * 16 + (d & 7) * 2);
      }
    }
  }

  // Operands of quarter q of a step whose scores come from half HB of K
  // buffer KB and whose P V uses half HB of V buffer VB: the K operands of
  // k-steps q*KQ .. q*KQ+KQ-1 and the V^T operands of the keys
  // 32*HB + 16*(q/2) + {4h..4h+3, 8+4h..8+4h+3} for dim blocks
  // (q%2)*VQ .. (q%2)*VQ+VQ-1.
  auto load_ops = [&](auto kb, auto vb, auto hb, auto qq) {
    constexpr int Q4 = decltype(qq)::value;
    constexpr int KOFF = decltype(kb)::value * TB + decltype(hb)::value * 32 * ROWB;
    constexpr int VOFF = decltype(vb)::value * TB + (decltype(hb)::value * 32 + 16 * (Q4 >> 1)) * ROWB;
    Ops o;
#pragma unroll
    for (int i = 0; i < KQ; ++i)
      o.k[i] = *reinterpret_cast<const lds_bf16x8*>(lds + k_off[Q4 * KQ + i] + KOFF);
#pragma unroll
    for (int i = 0; i < VQ; ++i) {
      const int db = (Q4 & 1) * VQ + i;
      const u32x2 lo = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + v_off[0][db] + VOFF)));
      const u32x2 hi = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + v_off[1][db] + VOFF)));
      o.v[i] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    return o;
  };

  // ------------------------------------------------------ per-block stages
  f32x16 oacc[2][C::NDB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) oacc[rb][i] = f32x16{};
  float m_ref[2] = {kNegInf, kNegInf};  // reference maximum per row block, log2 units
  float l_part[2] = {0.f, 0.f};         // this lane half's share of the row sums

  f32x16 sA[2], sB[2];          // S^T accumulators: even / odd blocks
  uint32_t pA[2][8], pB[2][8];  // bf16 P pairs: even / odd blocks

  // Block b needs a mask when it reaches past Nk or, causally, past the
  // wave's first query (blocks past the wave's last key are masked whole;
  // their K may be stale).  Accumulator register r of lane half h holds key
  // 32b + 4h + 8(r/4) + r%4; it is visible to row block rb iff that key is
  // <= lim(rb), i.e. iff 8(r/4) + r%4 <= lim(rb) - 32b - 4h.
  auto needs_mask = [&](int b) {
    const int kp = key_pos(b);
    return (kp + 32 > Nk) || (CAUSAL && kp + 31 > wq0 + off) || !admitted(b);
  };
  auto mask_room = [&](int b, int rb) {
    const int lim = CAUSAL ? min(Nk - 1, qi0 + 32 * rb + off) : Nk - 1;
    return admitted(b) ? lim - key_pos(b) - 4 * half : -(1 << 20);
  };

  // P = 2^(s*c - m) against the current reference (0 where masked) for
  // accumulator registers R0 .. R0+7 of a row block: bf16 pairs for the
  // matrix core, fp32 sum for l.
  // The eight values are independent until the final sum, and are written
  // stage by stage (all fma, all exp, pack, tree sum) so that in-order
  // issue never waits on one value's chain while matrix work is queued.
  auto exp8 = [&](auto masked, auto r0, const f32x16& s, float m_use, int room, uint32_t (&pk)[8],
                  float& lsum) {
    constexpr int R0 = decltype(r0)::value;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_fmaf(s[R0 + i], c, -m_use);
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = exp2_hw(p[i]);
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = R0 + i;
        p[i] = (8 * (r >> 2) + (r & 3) > room) ? 0.f : p[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2) pk[(R0 + i) >> 1] = pack_bf16x2(p[i], p[i + 1]);
    lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  };
  using R0c = std::integral_constant<int, 0>;
  using R8c = std::integral_constant<int, 8>;

  // A block whose P sum in some lane exceeds 2^8 (or is not finite: m = -inf
  // before the first visible key) takes the exact path: row maximum over the
  // visible keys, moved reference, l and O rescaled (O then holds the P V of
  // the blocks before b), P recomputed.  Every P then stays <= 2^8.
  auto fixup = [&](int b, const f32x16 (&sacc)[2], uint32_t (&pk)[2][8], float (&lsum)[2]) {
    if (__builtin_expect(wave_any(!(lsum[0] <= kSumBound) || !(lsum[1] <= kSumBound)), 0)) {
      [[unlikely]];
      consume(pk, lsum);
      products_done();  // O is read below
      const bool masked = needs_mask(b);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int room = masked ? mask_room(b, rb) : 31;
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          mx = (8 * (r >> 2) + (r & 3) > room) ? mx : fmaxf(mx, sacc[rb][r] * c);
        mx = max_across_halves(mx);
        const float m_new = fmaxf(m_ref[rb], mx);
        const float alpha = m_new != m_ref[rb] ? exp2_hw(m_ref[rb] - m_new) : 1.f;  // 0 from -inf
        l_part[rb] *= alpha;
        // O is rescaled one register at a time in place (read, multiply,
        // write back through a single temporary): written as a plain vector
        // product the compiler stages all of O in vector registers, and the
        // room that takes is then missing from the whole loop.
#pragma unroll
        for (int i = 0; i < C::NDB; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float x = oacc[rb][i][e];
            float t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t)
                         : "v"(alpha));
            oacc[rb][i][e] = x;
          }
        // The next products into O are inline assembly the compiler does not
        // see: give the rescaled accumulators their wait states here.
        asm volatile("s_nop 7" ::: "memory");
        m_ref[rb] = m_new;
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        lsum[rb] = 0.f;
        exp8(std::true_type{}, R0c{}, sacc[rb], m_use, room, pk[rb], lsum[rb]);
        exp8(std::true_type{}, R8c{}, sacc[rb], m_use, room, pk[rb], lsum[rb]);
      }
    }
    l_part[0] += lsum[0];
    l_part[1] += lsum[1];
  };

  // Quarter Q4 of a pipeline step around block b: the k-steps 2q, 2q+1 of
  // the scores of block b+1 (into s_nxt), the dim blocks 2(q%2), 2(q%2)+1 of
  // the P V of block b-1 for the keys of P pair group q/2, and eight of
  // block b's P values (row block q/2, registers 8(q%2)..8(q%2)+7).  The
  // three streams are independent; the instruction order is fixed here, as
  // eight groups of one matrix instruction and its share of the softmax:
  //   1 S(rb0,2q)  fma x4      2 PV(db0,rb0) fma x4
  //   3 S(rb1,2q)  exp x2      4 PV(db0,rb1) exp x2
  //   5 S(rb0,2q+1) exp x2, pack   6 PV(db1,rb0) exp x2, pack, add
  //   7 S(rb1,2q+1) pack, add x2   8 PV(db1,rb1) pack, add x5
  // Each exp result is read two groups later at the earliest (the one
  // wait state a transcendental result needs is always covered).
  auto quarter = [&](auto qq, const Ops& o, f32x16 (&s_nxt)[2], const f32x16 (&s_cur)[2],
                     uint32_t (&p_cur)[2][8], const uint32_t (&p_prv)[2][8], float (&lsum)[2]) {
    constexpr int Q4 = decltype(qq)::value;
    constexpr int RB = Q4 >> 1;
    constexpr int T = Q4 >> 1;
    constexpr int R0 = (Q4 & 1) * 8;
    constexpr int S0 = 2 * Q4;  // k-steps S0, S0+1
    constexpr int DB0 = (Q4 & 1) * 2;
    static_assert(D == 128, "explicit quarter schedule is written for d = 128");
    const bf16x8 b0 = __builtin_bit_cast(
        bf16x8, u32x4{p_prv[0][4 * T], p_prv[0][4 * T + 1], p_prv[0][4 * T + 2], p_prv[0][4 * T + 3]});
    const bf16x8 b1 = __builtin_bit_cast(
        bf16x8, u32x4{p_prv[1][4 * T], p_prv[1][4 * T + 1], p_prv[1][4 * T + 2], p_prv[1][4 * T + 3]});
    const f32x16& x = s_cur[RB];
    const float nm = -m_ref[RB];
    float p0, p1, p2, p3, p4, p5, p6, p7, t0, t1, t2, t3;
    uint32_t k0, k1, k2, k3;
#define FA_FMA(d, a) "v_fma_f32 " d ", " a ", %[c], %[nm]\n\t"
    // 1
    if constexpr (S0 == 0) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %[s], %[a], %[b], 0\n\t"
                   FA_FMA("%[p0]", "%[x0]") FA_FMA("%[p1]", "%[x1]") FA_FMA("%[p2]", "%[x2]") FA_FMA("%[p3]", "%[x3]")
                   : [s] "=&v"(s_nxt[0]), [p0] "=&v"(p0), [p1] "=&v"(p1), [p2] "=&v"(p2), [p3] "=&v"(p3)
                   : [a] "v"(o.k[0]), [b] "a"(qf[0][S0]), [x0] "v"(x[R0]), [x1] "v"(x[R0 + 1]),
                     [x2] "v"(x[R0 + 2]), [x3] "v"(x[R0 + 3]), [c] "s"(c), [nm] "v"(nm));
    } else {
      asm volatile("v_mfma_f32_32x32x16_bf16 %[s], %[a], %[b], %[s]\n\t"
                   FA_FMA("%[p0]", "%[x0]") FA_FMA("%[p1]", "%[x1]") FA_FMA("%[p2]", "%[x2]") FA_FMA("%[p3]", "%[x3]")
                   : [s] "+v"(s_nxt[0]), [p0] "=&v"(p0), [p1] "=&v"(p1), [p2] "=&v"(p2), [p3] "=&v"(p3)
                   : [a] "v"(o.k[0]), [b] "a"(qf[0][S0]), [x0] "v"(x[R0]), [x1] "v"(x[R0 + 1]),
                     [x2] "v"(x[R0 + 2]), [x3] "v"(x[R0 + 3]), [c] "s"(c), [nm] "v"(nm));
    }
    // 2
    asm volatile("v_mfma_f32_32x32x16_bf16 %[o], %[a], %[b], %[o]\n\t"
                 FA_FMA("%[p4]", "%[x4]") FA_FMA("%[p5]", "%[x5]") FA_FMA("%[p6]", "%[x6]") FA_FMA("%[p7]", "%[x7]")
                 : [o] "+a"(oacc[0][DB0]), [p4] "=&v"(p4), [p5] "=&v"(p5), [p6] "=&v"(p6), [p7] "=&v"(p7)
                 : [a] "v"(o.v[0]), [b] "v"(b0), [x4] "v"(x[R0 + 4]), [x5] "v"(x[R0 + 5]),
                   [x6] "v"(x[R0 + 6]), [x7] "v"(x[R0 + 7]), [c] "s"(c), [nm] "v"(nm));
    // 3
    if constexpr (S0 == 0) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %[s], %[a], %[b], 0\n\t"
                   "v_exp_f32 %[p0], %[p0]\n\tv_exp_f32 %[p1], %[p1]\n\t"
                   : [s] "=&v"(s_nxt[1]), [p0] "+v"(p0), [p1] "+v"(p1)
                   : [a] "v"(o.k[0]), [b] "a"(qf[1][S0]));
    } else {
      asm volatile("v_mfma_f32_32x32x16_bf16 %[s], %[a], %[b], %[s]\n\t"
                   "v_exp_f32 %[p0], %[p0]\n\tv_exp_f32 %[p1], %[p1]\n\t"
                   : [s] "+v"(s_nxt[1]), [p0] "+v"(p0), [p1] "+v"(p1)
                   : [a] "v"(o.k[0]), [b] "a"(qf[1][S0]));
    }
    // 4
    asm volatile("v_mfma_f32_32x32x16_bf16 %[o], %[a], %[b], %[o]\n\t"
                 "v_exp_f32 %[p2], %[p2]\n\tv_exp_f32 %[p3], %[p3]\n\t"
                 : [o] "+a"(oacc[1][DB0]), [p2] "+v"(p2), [p3] "+v"(p3)
                 : [a] "v"(o.v[0]), [b] "v"(b1));
    // 5
    asm volatile("v_mfma_f32_32x32x16_bf16 %[s], %[a], %[b], %[s]\n\t"
                 "v_exp_f32 %[p4], %[p4]\n\tv_exp_f32 %[p5], %[p5]\n\t"
                 "v_cvt_pk_bf16_f32 %[k0], %[p0], %[p1]\n\t"
                 : [s] "+v"(s_nxt[0]), [p4] "+v"(p4), [p5] "+v"(p5), [k0] "=&v"(k0)
                 : [a] "v"(o.k[1]), [b] "a"(qf[0][S0 + 1]), [p0] "v"(p0), [p1] "v"(p1));
    // 6
    asm volatile("v_mfma_f32_32x32x16_bf16 %[o], %[a], %[b], %[o]\n\t"
                 "v_exp_f32 %[p6], %[p6]\n\tv_exp_f32 %[p7], %[p7]\n\t"
                 "v_cvt_pk_bf16_f32 %[k1], %[p2], %[p3]\n\t"
                 "v_add_f32 %[t0], %[p0], %[p1]\n\t"
                 : [o] "+a"(oacc[0][DB0 + 1]), [p6] "+v"(p6), [p7] "+v"(p7), [k1] "=&v"(k1), [t0] "=&v"(t0)
                 : [a] "v"(o.v[1]), [b] "v"(b0), [p0] "v"(p0), [p1] "v"(p1), [p2] "v"(p2), [p3] "v"(p3));
    // 7
    asm volatile("v_mfma_f32_32x32x16_bf16 %[s], %[a], %[b], %[s]\n\t"
                 "v_cvt_pk_bf16_f32 %[k2], %[p4], %[p5]\n\t"
                 "v_add_f32 %[t1], %[p2], %[p3]\n\t"
                 "v_add_f32 %[t2], %[p4], %[p5]\n\t"
                 : [s] "+v"(s_nxt[1]), [k2] "=&v"(k2), [t1] "=&v"(t1), [t2] "=&v"(t2)
                 : [a] "v"(o.k[1]), [b] "a"(qf[1][S0 + 1]), [p2] "v"(p2), [p3] "v"(p3), [p4] "v"(p4),
                   [p5] "v"(p5));
    // 8
    asm volatile("v_mfma_f32_32x32x16_bf16 %[o], %[a], %[b], %[o]\n\t"
                 "v_cvt_pk_bf16_f32 %[k3], %[p6], %[p7]\n\t"
                 "v_add_f32 %[t3], %[p6], %[p7]\n\t"
                 "v_add_f32 %[t0], %[t0], %[t1]\n\t"
                 "v_add_f32 %[t2], %[t2], %[t3]\n\t"
                 "v_add_f32 %[t0], %[t0], %[t2]\n\t"
                 "v_add_f32 %[l], %[l], %[t0]\n\t"
                 : [o] "+a"(oacc[1][DB0 + 1]), [k3] "=&v"(k3), [t3] "=&v"(t3), [t0] "+v"(t0),
                   [t2] "+v"(t2), [l] "+v"(lsum[RB])
                 : [a] "v"(o.v[1]), [b] "v"(b1), [p6] "v"(p6), [p7] "v"(p7), [t1] "v"(t1));
#undef FA_FMA
    p_cur[RB][R0 / 2] = k0;
    p_cur[RB][R0 / 2 + 1] = k1;
    p_cur[RB][R0 / 2 + 2] = k2;
    p_cur[RB][R0 / 2 + 3] = k3;
    // The LDS reads of the next quarter go first in the quarter.
    __builtin_amdgcn_sched_group_barrier(0x100, KQ + 2 * VQ, 0);
  };

  // Masking of block b after the fact, per row block: where every row sees
  // every key (a causal diagonal block is so for one of its two row blocks)
  // P stands; where no row sees any key (the other row block of the second
  // diagonal block, the block after the wave's last key, keys past Nk) P and
  // the P sums are cleared without any arithmetic; otherwise P is formed
  // again from the scores with the keys past lim(rb) cleared.  Whatever a
  // stale score produced is dropped.
  auto apply_mask = [&](int b, const f32x16 (&sacc)[2], uint32_t (&pk)[2][8], float (&lsum)[2]) {
    consume(pk, lsum);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int room = mask_room(b, rb);
      // register 15 holds key 27 (+4 in the upper lane half, already in room)
      if (!wave_any(room < 27)) continue;
      lsum[rb] = 0.f;
      if (!wave_any(room >= 0)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pk[rb][i] = 0u;
        continue;
      }
      exp8(std::true_type{}, R0c{}, sacc[rb], m_ref[rb], room, pk[rb], lsum[rb]);
      exp8(std::true_type{}, R8c{}, sacc[rb], m_ref[rb], room, pk[rb], lsum[rb]);
    }
  };

  // One pipeline step around block b: four quarters, each using operands
  // read during the one before; the last reads the first operands of the
  // next step (K buffer NKB, V buffer NVB, half NHB).  Masking and the
  // exact-maximum path follow the quarters as rare branches.
  auto step = [&](auto kb, auto vb, auto hb, auto nkb, auto nvb, auto nhb, int b, Ops& ops,
                  f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], uint32_t (&p_cur)[2][8],
                  const uint32_t (&p_prv)[2][8]) {
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    using Q3 = std::integral_constant<int, 3>;
    float lsum[2] = {0.f, 0.f};
    Ops n1 = load_ops(kb, vb, hb, Q1{});
    quarter(Q0{}, ops, s_nxt, s_cur, p_cur, p_prv, lsum);
    __builtin_amdgcn_sched_barrier(0);
    Ops n2 = load_ops(kb, vb, hb, Q2{});
    quarter(Q1{}, n1, s_nxt, s_cur, p_cur, p_prv, lsum);
    __builtin_amdgcn_sched_barrier(0);
    Ops n3 = load_ops(kb, vb, hb, Q3{});
    quarter(Q2{}, n2, s_nxt, s_cur, p_cur, p_prv, lsum);
    __builtin_amdgcn_sched_barrier(0);
    ops = load_ops(nkb, nvb, nhb, Q0{});
    quarter(Q3{}, n3, s_nxt, s_cur, p_cur, p_prv, lsum);
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_expect(needs_mask(b), 0)) {
      [[unlikely]];
      apply_mask(b, s_cur, p_cur, lsum);
    }
    fixup(b, s_cur, p_cur, lsum);
  };

  // Tile iteration j (buffer U = j % kNBuf) first requests the K tile four
  // positions and the V tile three positions ahead in the stream (into the
  // buffers of K tile j and V tile j-1, whose last readers passed the
  // previous barrier; past the item's end these are the next item's first
  // tiles), then runs the steps around blocks 2j+1 and 2j+2, which read K
  // tile j+1 and V tile j (and, ahead, the first operands of K tile j+2 and
  // V tile j+1), and finally waits for all but its own requests, so the
  // tiles of positions j+3 (K) and j+2 (V) are in place for iteration j+1.
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  Ops ops;
  int r_cur = 0;  // round of the item being computed (streaming)
  auto iteration = [&](auto u, int j, bool tail) {
    constexpr int U = decltype(u)::value;
    using KB = std::integral_constant<int, (U + 1) % kNBuf>;
    using VB = std::integral_constant<int, U>;
    using NKB = std::integral_constant<int, (U + 2) % kNBuf>;
    using NVB = std::integral_constant<int, (U + 1) % kNBuf>;
    paranoid_sync();
    bool ik, iv;
    if (!tail) {  // the item's own tiles only
      ik = j + 4 < n_tiles;
      iv = j + 3 < n_tiles;
      if (ik) issue(reinterpret_cast<const char*>(K + kbase), U * TB, j + 4);
      if (iv) issue(reinterpret_cast<const char*>(V + kbase), VREG + ((U + 3) % kNBuf) * TB, j + 3);
    } else {  // the item's last positions: its own tiles or the next item's first
      ik = issue_k(std::integral_constant<int, U>{}, j + 4);
      iv = issue_v(std::integral_constant<int, (U + 3) % kNBuf>{}, j + 3);
    }
    paranoid_sync();
    if (j < njw) {
      step(KB{}, VB{}, H0{}, KB{}, VB{}, H1{}, 2 * j + 1, ops, sB, sA, pB, pA);
      step(KB{}, VB{}, H1{}, NKB{}, NVB{}, H0{}, 2 * j + 2, ops, sA, sB, pA, pB);
    }
    wait_vm<C::IPW>(ik, iv);
    __syncthreads();
  };

  // ------------------------------------------------------------- main loop
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  // Requests in order: Q (above), K and V of positions 0 and 1, K of
  // position 2.  At the first item's start all of them are in place; a
  // barrier, and then the requests of positions 3 (K) and 2 (V), as a tile
  // iteration would have made them.
  paranoid_sync();
  if constexpr (STREAM) find_next(1);
  issue_k(B0{}, 0);
  issue_v(B0{}, 0);
  issue_k(B1{}, 1);
  issue_v(B1{}, 1);
  issue_k(B2{}, 2);

  for (bool first = true;; first = false) {
    paranoid_sync();
    // The item's Q has landed once nothing is in flight (the first item's
    // was requested above, a later item's at the end of the item before).
    // Redefining qf here keeps the compiler from placing waits for those
    // loads inside the walk, where the tile copies in flight would turn them
    // into stalls; on every path to the walk qf is redefined here.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s = 0; s < C::KS; ++s) asm volatile("" : "+a"(qf[rb][s]));
    if (first) {
      __syncthreads();
      issue_k(B3{}, 3);
      issue_v(B2{}, 2);
    }
    if constexpr (STREAM) {
      if (!first) {
        // The next item: its K tiles 0-2 and V tiles 0-1 are in place (the
        // last barrier published them), K tile 3 and V tile 2 are in flight.
        set_dense_item((int)item_at(r_cur));
        set_rows();
        set_wave_blocks();
        n_tiles = n_cand;
        n_pos = (n_tiles + kNBuf - 1) / kNBuf * kNBuf;
        find_next(r_cur + 1);
      }
    }
    if (n_tiles > 0) {
      if (nbw > 0) {  // block 0 and the scores of block 1 before the first tile iteration
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          f32x16(&sacc)[2] = hb ? sB : sA;
#pragma unroll
          for (int s = 0; s < C::KS; ++s) {
            const bf16x8 a = *reinterpret_cast<const lds_bf16x8*>(lds + k_off[s] + hb * 32 * ROWB);
            if (s == 0) {
              qk_first(sacc[0], a, qf[0][s]);
              qk_first(sacc[1], a, qf[1][s]);
            } else {
              qk_next(sacc[0], a, qf[0][s]);
              qk_next(sacc[1], a, qf[1][s]);
            }
          }
        }
        products_done();
        // Block 0 sets the reference: its exact row maximum over the visible
        // keys (O and l are still zero, so nothing is rescaled).
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          int room = mask_room(0, rb);
          // opaque to the compiler: its compares against room would
          // otherwise be hoisted out of the item loop as 64-bit lane masks
          // and occupy scalar registers across the whole walk
          asm volatile("" : "+v"(room));
          float mx = kNegInf;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            mx = (8 * (r >> 2) + (r & 3) > room) ? mx : fmaxf(mx, sA[rb][r] * c);
          m_ref[rb] = max_across_halves(mx);
          const float m_use = m_ref[rb] == kNegInf ? 0.f : m_ref[rb];
          exp8(std::true_type{}, R0c{}, sA[rb], m_use, room, pA[rb], l_part[rb]);
          exp8(std::true_type{}, R8c{}, sA[rb], m_use, room, pA[rb], l_part[rb]);
        }
      }
      // Every wave has read K tile 0 before the first iteration requests
      // the tile four positions ahead into its buffer.
      __syncthreads();
      if (nbw > 0) ops = load_ops(B1{}, B0{}, H0{}, std::integral_constant<int, 0>{});
      for (int j = 0; j < n_pos; j += kNBuf) {
        const bool tail = STREAM && j + kNBuf == n_pos;  // the last group reaches into the next item
        iteration(B0{}, j, tail);
        if (!STREAM && j + 1 >= n_pos) break;
        iteration(B1{}, j + 1, tail);
        if (!STREAM && j + 2 >= n_pos) break;
        iteration(B2{}, j + 2, tail);
        if (!STREAM && j + 3 >= n_pos) break;
        iteration(B3{}, j + 3, tail);
      }
    }

    products_done();  // the epilogue reads O

    // Epilogue: one division per row, O in bf16, LSE = ln2 * (m + log2 l).
    if constexpr (STREAM) {
      // The next item's Q is requested first, so that its latency overlaps
      // this epilogue (the current Q is no longer read).
      const bool more = valid_round(r_cur + 1);
      if (more) {
        const int nx = (int)item_at(r_cur + 1);
        load_q(qf, (size_t)(nx % BH) * Nq * D, (n_qtiles - 1 - nx / BH) * kBR + wave * 64);
      }
      __builtin_amdgcn_sched_barrier(0);
      // The next item's tiles fill the K buffers and V buffers 0-2; V buffer
      // 3 (its last reader passed the last barrier, and the next item's first
      // iteration refills it only after a barrier) and the 16 KB after it
      // give each wave 8 KB: O leaves 32 rows at a time, written row-major
      // with the 16-byte chunks of row r at slots c ^ (r % 16), read back as
      // whole rows and stored with 16-byte non-temporal writes, 1 KB
      // contiguous per wave instruction.  O is not read again by the kernel;
      // as ordinary writes its lines took L2 room from the K/V tiles the
      // other workgroups of the XCD re-read (3-5% of the causal rate).
      const size_t qb = (size_t)(((int)item_at(r_cur)) % BH) * Nq * D;
      lds_char* const otile = lds + VREG + 3 * TB + wave * 32 * ROWB;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float l_tot = sum_across_halves(l_part[rb]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const u32x2 w = {pack_bf16x2(oacc[rb][db][4 * g4] * inv, oacc[rb][db][4 * g4 + 1] * inv),
                             pack_bf16x2(oacc[rb][db][4 * g4 + 2] * inv, oacc[rb][db][4 * g4 + 3] * inv)};
            const int chunk = 4 * db + g4;  // dims 32db + 8g .. +7; this lane half holds +4h .. +4h+3
            *reinterpret_cast<lds_u32x2*>(otile + col * ROWB + ((chunk ^ (col & 15)) * 16) + 8 * half) = w;
          }
        const int row = qi0 + 32 * rb;
        if (half == 0 && row < Nq)
          LSE[(size_t)(((int)item_at(r_cur)) % BH) * Nq + row] =
              l_tot > 0.f ? (m_ref[rb] + log2_hw(l_tot)) * kLn2 : kNegInf;
        // same wave: program order orders these reads after the writes above
        constexpr int kRowsPerStore = 64 * 16 / ROWB;  // rows covered by 64 lanes x 16 B
#pragma unroll
        for (int it = 0; it < 32 / kRowsPerStore; ++it) {
          const int r = it * kRowsPerStore + lane / C::CPR;
          const int cc = lane % C::CPR;
          const u32x4 w = *reinterpret_cast<const lds_u32x4*>(otile + r * ROWB + ((cc ^ (r & 15)) * 16));
          const int grow = wq0 + 32 * rb + r;
          if (grow < Nq) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(O + qb + (size_t)grow * q_rs + cc * 8));
        }
        // the second row block reuses the region: its writes follow these
        // reads in program order, and LDS operations of a wave complete in order
      }
    } else {
      // O leaves through LDS (free after the last barrier): each wave writes
      // its 64 x D tile row-major into its own 16 KB region, with the 16-byte
      // chunks of row r at slots c ^ (r % 16), then reads whole rows back and
      // stores them with 16-byte non-temporal writes, 1 KB contiguous per
      // wave instruction.
      lds_char* const otile = lds + wave * 64 * ROWB;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * rb + col;  // row within the wave's tile
        const float l_tot = sum_across_halves(l_part[rb]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const u32x2 w = {pack_bf16x2(oacc[rb][db][4 * g4] * inv, oacc[rb][db][4 * g4 + 1] * inv),
                             pack_bf16x2(oacc[rb][db][4 * g4 + 2] * inv, oacc[rb][db][4 * g4 + 3] * inv)};
            const int chunk = 4 * db + g4;  // dims 32db + 8g .. +7; this lane half holds +4h .. +4h+3
            *reinterpret_cast<lds_u32x2*>(otile + r * ROWB + ((chunk ^ (r & 15)) * 16) + 8 * half) = w;
          }
        const int row = qi0 + 32 * rb;
        if (half == 0 && row < Nq)
          LSE[lse_base + row] = l_tot > 0.f ? (m_ref[rb] + log2_hw(l_tot)) * kLn2 : kNegInf;
      }
      // Same wave wrote the region, so program order is enough between the
      // writes and these reads.
      constexpr int kRowsPerStore = 64 * 16 / ROWB;  // rows covered by 64 lanes x 16 B
#pragma unroll
      for (int it = 0; it < 64 / kRowsPerStore; ++it) {
        const int r = it * kRowsPerStore + lane / C::CPR;
        const int cc = lane % C::CPR;
        const u32x4 w = *reinterpret_cast<const lds_u32x4*>(otile + r * ROWB + ((cc ^ (r & 15)) * 16));
        const int row = wq0 + r;
        if (row < Nq) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(O + qbase + (size_t)row * q_rs + cc * 8));
      }
      break;
    }
    // Fresh state for the next item.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int i = 0; i < C::NDB; ++i) oacc[rb][i] = f32x16{};
      m_ref[rb] = kNegInf;
      l_part[rb] = 0.f;
    }
    if (!valid_round(++r_cur)) break;
  }
}

template <int D, bool CAUSAL, bool VARLEN, bool SPARSE>
hipError_t launch(const FwdArgs& a) {
  const int n_qtiles = (int)(((long long)a.Nq + kBR - 1) / kBR);
  const int BH = a.B * a.H;
  // Scores enter the exponent as s * c (log2 units); masking acts on P,
  // so c may have either sign or be zero.
  const float c = a.scale * kLog2e;
  const int n_items = n_qtiles * BH;
  // Dense: one workgroup per CU (the LDS and registers of one workgroup
  // fill a CU), each streaming every G-th item.  Varlen and block-sparse:
  // one workgroup per item.
  int G = n_items;
  if constexpr (!VARLEN && !SPARSE) {
    int cus = 0;
    const hipError_t e = cu_count(a.stream, &cus);
    if (e != hipSuccess) return e;
    G = min(n_items, cus);
  }
  const dim3 grid = VARLEN ? dim3((unsigned)(n_qtiles * a.H), (unsigned)a.B) : dim3((unsigned)G);
  const dim3 block(kThreads);
  void* args[] = {(void*)&a.q,     (void*)&a.k,    (void*)&a.v,  (void*)&a.o,       (void*)&a.lse,
                  (void*)&BH,      (void*)&a.Nq,   (void*)&a.Nk, (void*)&c,         (void*)&n_qtiles,
                  (void*)&a.cu_q,  (void*)&a.cu_k, (void*)&a.H,  (void*)&a.total_q, (void*)&a.bmask,
                  (void*)&a.nqb,   (void*)&a.nkb,  (void*)&n_items};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, CAUSAL, VARLEN, SPARSE>),
                         grid, block, args, 0, a.stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d != 128) return launch_fwd_bf16_d64(a);
  if (a.cu_q) return a.causal ? launch<128, true, true, false>(a) : launch<128, false, true, false>(a);
  if (a.bmask) return a.causal ? launch<128, true, false, true>(a) : launch<128, false, false, true>(a);
  return a.causal ? launch<128, true, false, false>(a) : launch<128, false, false, false>(a);
}

long long fwd_bf16_grid(int B, int H, int Nq) {
  return (((long long)Nq + kBR - 1) / kBR) * B * H;
}

}  // namespace fa
