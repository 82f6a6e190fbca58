// bwd_bf16.hip — gradients of exact attention by recomputation (bf16 inputs,
// fp32 gradients).
//
// The forward pass keeps only O and the row statistic LSE; the backward pass
// rebuilds each block of scores and probabilities on chip from Q, K and LSE
// instead of storing the N x N matrices (AI圣经13 review §03,
// "recomputation"; explainer §3).  With S = scale Q K^T and P = exp(S - LSE):
//
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = rowsum(dO * O)_i,
//     dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels: a row pass (D, and LSE in log2 units), one with K and V
// fixed per wave that walks the query blocks (dK, dV), one with Q and dO
// fixed per wave that walks the key blocks (dQ).  The last two recompute S
// and dP each (7 products per block pair instead of 5) so that no gradient
// needs atomic accumulation across workgroups.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, wave64): lane l holds
// A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32]; accumulator register
// r holds D[8*(r/4) + 4*(l/32) + r%4][l%32].  Products whose k index runs
// over a block's rows (dV, dK, dQ) take P or dS straight from the
// accumulators as the B operand and read the A operand from LDS with the
// transposing read ds_read_b64_tr_b16, addressed so that the k order matches
// the rows those accumulator registers hold.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRows = 32;                  // rows of a fixed block per wave, and of a moving block
constexpr int kFixed = kWaves * kRows;     // fixed rows per workgroup
constexpr int kDkdvBufs = 8;               // LDS buffers of the moving Q / dO blocks (dK/dV)
constexpr int kDkdvAhead = kDkdvBufs / 2;  // blocks staged ahead; blocks per barrier
constexpr int kDqBufs = 4;                 // LDS buffers of the moving K / V blocks (dQ)

// LDS slot of 16-byte chunk c of tile row r (the forward's permutation):
// a chunk read across 32 rows and the transposing reads are conflict-free.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
}

template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;           // bytes per row
  static constexpr int BYTES = kRows * ROWB;   // one 32-row tile
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int PER_THREAD = kRows * CPR / kThreads;  // chunks per thread per tile
  static constexpr int KS = D / 16;            // k-steps over d
  static constexpr int NDB = D / 32;           // 32-wide blocks of d
};

// LDS operands of the products.  Row-major operand of one k-step: lane holds
// row (lane%32), dims 16 s + 8 (lane/32) .. +7.  Transposed operand of dim
// block db over 16 rows: lane holds dim 32 db + lane%32 of the rows
// {4h .. 4h+3, 8+4h .. 8+4h+3} (h = lane/32) -- the rows accumulator
// registers 8t .. 8t+7 of a 32-row block hold -- read with the transposing
// ds_read_b64_tr_b16.  Both are read through per-lane addresses formed once
// per block: lane_addr() adds a lane's offset within a tile to the tile's
// base and hides the sum from re-association, so that constant
// displacements added afterwards (the dO tile after the Q tile, the second
// 16 rows of a block) fold into the reads' immediate offsets instead of
// costing an add per read.
template <int D>
struct OpOffsets {
  uint32_t row[Tile<D>::KS];     // row operand of k-step s
  uint32_t tr[Tile<D>::NDB][2];  // transposed operand of dim block db, read cc, rows 0..15
};
template <int D>
__device__ __forceinline__ OpOffsets<D> op_offsets(int lane) {
  OpOffsets<D> o;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < Tile<D>::KS; ++s) o.row[s] = (uint32_t)(r * Tile<D>::ROWB + swz<D>(r, 2 * s + h) * 16);
#pragma unroll
  for (int db = 0; db < Tile<D>::NDB; ++db) {
    const int dim = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int row = 8 * cc + 4 * h + ((lane & 15) >> 2);
      o.tr[db][cc] = (uint32_t)(row * Tile<D>::ROWB + swz<D>(row, dim >> 3) * 16 + (dim & 7) * 2);
    }
  }
  return o;
}
__device__ __forceinline__ uint32_t lane_addr(const lds_char* tile, uint32_t off) {
  uint32_t a = (uint32_t)(size_t)tile + off;
  asm volatile("" : "+v"(a));
  return a;
}
__device__ __forceinline__ bf16x8 row_at(uint32_t a, int disp) {
  return *reinterpret_cast<const lds_bf16x8*>((size_t)(a + disp));
}
// Transposed operand from the two read addresses of a dim block; disp
// selects the tile (Q or dO, K or V) and the 16-row half (+16 rows).
__device__ __forceinline__ bf16x8 tr_at(const uint32_t (&a)[2], int disp) {
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)(a[0] + disp)));
  const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)(a[1] + disp)));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Matrix products written as single instructions so that the score products
// land in vector registers (the row work reads them) and the gradient
// accumulators stay in accumulation registers for the whole pass (as a
// compiled product the compiler moves them between register files every
// block).  The compiler does not see these as matrix instructions, so it
// inserts none of the wait states their results need: each pause below
// takes the registers it guards as operands, which puts every later reader
// of them after the pause.
// The score products take their fixed B operand (the rows a workgroup keeps
// for the whole pass) from accumulation registers: held there, it is never
// copied into vector registers by the vector unit just before a product
// reads it (a hazard the compiler does not guard for these statements).
__device__ __forceinline__ void mm_first(f32x16& d, bf16x8 a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mm_next(f32x16& d, bf16x8 a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mm_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Zeroed accumulators, produced in accumulation registers by a product of
// zero operands: every value the accumulators take is then defined there, and
// the compiler keeps them there across the loop instead of holding them in
// vector registers and copying them over around each product.
template <int N>
__device__ __forceinline__ void zero_acc(f32x16 (&a)[N]) {
  bf16x8 z = {};
  asm volatile("s_nop 4" : "+v"(z));  // the zeros are written by the vector unit
#pragma unroll
  for (int i = 0; i < N; ++i)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(a[i]) : "v"(z));
}

// Before vector instructions read the two score products.
__device__ __forceinline__ void pause_scores(f32x16& a, f32x16& b) {
  asm volatile("s_nop 15\n\ts_nop 15" : "+v"(a), "+v"(b));
}
// Before the accumulators are read out, after the last product into them.
template <int N>
__device__ __forceinline__ void pause_acc(f32x16 (&a)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(a[i]));
}
// Before a product reads B operands the vector unit has just written.
__device__ __forceinline__ void pause_operands(bf16x8 (&a)[2]) {
  asm volatile("s_nop 4" : "+v"(a[0]), "+v"(a[1]));
}
__device__ __forceinline__ void pause_operands(bf16x8 (&a)[2], bf16x8 (&b)[2]) {
  asm volatile("s_nop 4" : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]));
}

// Returns the tile pointers unchanged, but only after every matrix
// instruction issued above it: loads addressed through the results are not
// moved ahead of those products (which would hold their registers longer).
__device__ __forceinline__ void after_products(const lds_char*& a, const lds_char*& b) {
  asm volatile("" : "+s"(a), "+s"(b));
}
template <int N>
__device__ __forceinline__ void after_products(uint32_t (&a)[N][2]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(a[i][0]), "+v"(a[i][1]));
}

// Accumulator registers 8t .. 8t+7 packed to bf16 as a B operand.
__device__ __forceinline__ bf16x8 pack_b(const float (&x)[16], int t) {
  return __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(x[8 * t], x[8 * t + 1]),
                                          pack_bf16x2(x[8 * t + 2], x[8 * t + 3]),
                                          pack_bf16x2(x[8 * t + 4], x[8 * t + 5]),
                                          pack_bf16x2(x[8 * t + 6], x[8 * t + 7])});
}

// 16 bytes of row min(row, n-1) of a [n, D] bf16 matrix, dims 16 s + 8 h ..
template <int D>
__device__ __forceinline__ bf16x8 load_row_op(const bf16* base, int row, int n, int lane, int s) {
  const int h = lane >> 5;
  return *reinterpret_cast<const bf16x8*>(base + (size_t)min(row, n - 1) * D + 16 * s + 8 * h);
}

// Stage a 32-row tile (rows r0 .. r0+31, clamped to n-1) of a [n, D] matrix:
// fetch into registers, then write them to LDS.
template <int D>
struct Stager {
  u32x4 v[Tile<D>::PER_THREAD];
  __device__ __forceinline__ void fetch(const bf16* base, int r0, int n, int tid) {
#pragma unroll
    for (int i = 0; i < Tile<D>::PER_THREAD; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / Tile<D>::CPR, ch = c % Tile<D>::CPR;
      v[i] = *reinterpret_cast<const u32x4*>(base + (size_t)min(r0 + r, n - 1) * D + ch * 8);
    }
  }
  __device__ __forceinline__ void store(lds_char* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < Tile<D>::PER_THREAD; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / Tile<D>::CPR, ch = c % Tile<D>::CPR;
      *reinterpret_cast<lds_u32x4*>(tile + r * Tile<D>::ROWB + swz<D>(r, ch) * 16) = v[i];
    }
  }
};

// ---------------------------------------------------------------- row pass
// D_i = sum_d dO[i][d] O[i][d] (fp32), and LSE in log2 units, with rows that
// saw no key (LSE = -inf) mapped to +inf so that every P of theirs is 0.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_kernel(const bf16* __restrict__ O,
                                                            const bf16* __restrict__ dO,
                                                            const float* __restrict__ LSE,
                                                            float* __restrict__ lse2,
                                                            float* __restrict__ Dv, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long row = (long long)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + sub * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + sub * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc += bf16_lo(a[i]) * bf16_lo(b[i]) + bf16_hi(a[i]) * bf16_hi(b[i]);
  }
  acc = D == 128 ? sum_row16(acc) : sum_row8(acc);
  if (row < rows && sub == 0) {
    Dv[row] = acc;
    const float l = LSE[row];
    lse2[row] = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
  }
}

// -------------------------------------------------------------- dK and dV
// Workgroup: 4 waves x 32 keys; key tile kt = blockIdx.x / BH (early keys,
// which the most queries see, first), (b, h) = blockIdx.x % BH.  The query
// blocks stream through LDS (Q, dO, LSE2, D), double-buffered.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ Dv,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int Nq, int Nk, float c, float scale) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[kDkdvBufs * (2 * T::BYTES + 2 * kRows * 4)];
  lds_char* const lds = (lds_char*)smem;
  auto q_tile = [&](int buf) { return lds + buf * (2 * T::BYTES + 256); };
  auto do_tile = [&](int buf) { return q_tile(buf) + T::BYTES; };
  auto st_tile = [&](int buf) { return q_tile(buf) + 2 * T::BYTES; };  // lse2[32], D[32]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int kt = (int)(blockIdx.x / BH), bh = (int)(blockIdx.x % BH);
  const int off = Nk - Nq;
  const int k0w = kt * kFixed + wave * kRows;  // this wave's first key
  const bf16* Qh = Q + (size_t)bh * Nq * D;
  const bf16* dOh = dO + (size_t)bh * Nq * D;
  const float* l2h = lse2 + (size_t)bh * Nq;
  const float* Dh = Dv + (size_t)bh * Nq;

  // Query blocks that see any key of the workgroup.  Every wave takes every
  // one of them: a block that sees none of the wave's keys lies above the
  // diagonal for all of them, so the causal mask zeroes its P and dS (the
  // few blocks this costs are cheaper than a branch around the body, across
  // which the compiler moves the accumulators).
  const int n_qb = (Nq + kRows - 1) / kRows;
  const int qb_first = CAUSAL ? max(0, kt * kFixed - off) / kRows : 0;

  // Fixed operands: K and V rows of this wave's keys as B operands.
  bf16x8 kf[T::KS], vf[T::KS];
#pragma unroll
  for (int s = 0; s < T::KS; ++s) {
    kf[s] = load_row_op<D>(K + (size_t)bh * Nk * D, k0w + col, Nk, lane, s);
    vf[s] = load_row_op<D>(V + (size_t)bh * Nk * D, k0w + col, Nk, lane, s);
  }
  f32x16 dk[T::NDB], dv[T::NDB];
  zero_acc(dk);
  zero_acc(dv);

  Stager<D> sq, sd;
  float st = 0.f;  // this thread's lse2 or D value of the next block (threads 0..63)
  const OpOffsets<D> oo = op_offsets<D>(lane);
  auto fetch = [&](int qb) {
    sq.fetch(Qh, qb * kRows, Nq, tid);
    sd.fetch(dOh, qb * kRows, Nq, tid);
    if (tid < 2 * kRows) {
      const int r = qb * kRows + (tid & (kRows - 1));
      st = r < Nq ? (tid < kRows ? l2h[r] : Dh[r]) : (tid < kRows ? __builtin_huge_valf() : 0.f);
    }
  };
  auto store = [&](int buf) {
    sq.store(q_tile(buf), tid);
    sd.store(do_tile(buf), tid);
    if (tid < 2 * kRows) reinterpret_cast<__attribute__((address_space(3))) float*>(st_tile(buf))[tid] = st;
  };

  // kDkdvBufs LDS buffers; block j (counted from qb_first) uses buffer
  // j % kDkdvBufs.  With A = kDkdvAhead = kDkdvBufs / 2, block qb+A is
  // fetched into registers during block qb-1 and written to LDS in the
  // middle of block qb (between its last LDS reads and its softmax, when the
  // LDS is otherwise idle).  A barrier follows every A-th block (j % A =
  // A-1): block j writes buffer (j+A) % kDkdvBufs, last read by block j-A,
  // and reads buffer j % kDkdvBufs, written in block j-A; of the A blocks
  // j-A .. j-1 exactly one ends with a barrier, which lies after block j-A's
  // accesses and before block j's.
  if (qb_first < n_qb) {
    for (int i = 0; i < kDkdvAhead && qb_first + i < n_qb; ++i) {
      fetch(qb_first + i);
      store(i);
    }
    if (qb_first + kDkdvAhead < n_qb) fetch(qb_first + kDkdvAhead);
    __syncthreads();
  }
  for (int qb = qb_first; qb < n_qb; ++qb) {
    const int buf = (qb - qb_first) & (kDkdvBufs - 1);
    paranoid_sync();
    {
      const lds_char* qt = q_tile(buf);
      const lds_char* dt = do_tile(buf);
      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys:
      // lane = key (column), register r = query 8(r/4) + 4 half + r%4.
      // All operands first (the block's lse2 and D values with them), then
      // the products.
      const auto* stp = reinterpret_cast<const __attribute__((address_space(3))) float*>(st_tile(buf));
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        l4[g] = *reinterpret_cast<const lds_f32x4*>(stp + 8 * g + 4 * half);
        d4[g] = *reinterpret_cast<const lds_f32x4*>(stp + kRows + 8 * g + 4 * half);
      }
      bf16x8 qa[T::KS], da[T::KS];
#pragma unroll
      for (int s = 0; s < T::KS; ++s) {
        const uint32_t a = lane_addr(qt, oo.row[s]);
        qa[s] = row_at(a, 0);
        da[s] = row_at(a, T::BYTES);  // the dO tile follows the Q tile
      }
      f32x16 S, dP;
      mm_first(S, qa[0], kf[0]);
      mm_first(dP, da[0], vf[0]);
#pragma unroll
      for (int s = 1; s < T::KS; ++s) {
        mm_next(S, qa[s], kf[s]);
        mm_next(dP, da[s], vf[s]);
      }
      // transposed operands of the first 16 queries, read during the wait
      uint32_t ta[T::NDB][2];
      bf16x8 tdo[T::NDB], tq[T::NDB];
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) {
        ta[db][0] = lane_addr(qt, oo.tr[db][0]);
        ta[db][1] = lane_addr(qt, oo.tr[db][1]);
        tdo[db] = tr_at(ta[db], T::BYTES);
        tq[db] = tr_at(ta[db], 0);
      }
      pause_scores(S, dP);
      if (qb + kDkdvAhead < n_qb) {
        // buffer (buf + A) % kDkdvBufs was last read A blocks ago, before a barrier
        store((buf + kDkdvAhead) & (kDkdvBufs - 1));
        if (qb + kDkdvAhead + 1 < n_qb) fetch(qb + kDkdvAhead + 1);
      }
      float P[16], dS[16];
      const int key = k0w + col;
      // P and dS; only blocks that cross this wave's diagonal test keys
      // (a uniform branch around vector work only: no product inside).
      auto softmax = [&](auto masked) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            float p = exp2_hw(S[r] * c - l4[g][i]);
            if constexpr (decltype(masked)::value)
              if (key > qb * kRows + 8 * g + 4 * half + i + off) p = 0.f;
            P[r] = p;
            dS[r] = p * (dP[r] - d4[g][i]);
          }
        }
      };
      if (CAUSAL && k0w + kRows - 1 > qb * kRows + off)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
      // dV^T += dO^T P and dK^T += Q^T dS over the block's 32 queries.
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        pb[t] = pack_b(P, t);
        sb[t] = pack_b(dS, t);
      }
      pause_operands(pb, sb);
      // The first 16 queries' products; the last 16 queries' operands are
      // read while the second half of them runs.
      constexpr int H1 = T::NDB / 2;
#pragma unroll
      for (int db = 0; db < H1; ++db) {
        mm_acc(dv[db], tdo[db], pb[0]);
        mm_acc(dk[db], tq[db], sb[0]);
      }
      after_products(ta);
      bf16x8 udo[T::NDB], uq[T::NDB];
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) {
        udo[db] = tr_at(ta[db], T::BYTES + 16 * T::ROWB);
        uq[db] = tr_at(ta[db], 16 * T::ROWB);
      }
#pragma unroll
      for (int db = H1; db < T::NDB; ++db) {
        mm_acc(dv[db], tdo[db], pb[0]);
        mm_acc(dk[db], tq[db], sb[0]);
      }
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) {
        mm_acc(dv[db], udo[db], pb[1]);
        mm_acc(dk[db], uq[db], sb[1]);
      }
    }
    if ((qb - qb_first) % kDkdvAhead == kDkdvAhead - 1 && qb + 1 < n_qb) __syncthreads();
    paranoid_sync();
  }

  // dK^T / dV^T accumulators: lane = key, register r of dim block db =
  // dim 32 db + 8(r/4) + 4 half + r%4.
  pause_acc(dk);
  pause_acc(dv);
  const int key = k0w + col;
  if (key < Nk) {
    float* dKr = dK + ((size_t)bh * Nk + key) * D;
    float* dVr = dV + ((size_t)bh * Nk + key) * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        *reinterpret_cast<f32x4*>(dKr + d0) =
            f32x4{dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale, dk[db][4 * g + 2] * scale,
                  dk[db][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(dVr + d0) =
            f32x4{dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
      }
  }
}

// -------------------------------------------------------------------- dQ
// Workgroup: 4 waves x 32 queries; query tile qt = n_qt - 1 - blockIdx.x / BH
// (late queries, which see the most keys, first).  The key blocks stream
// through four LDS buffers (K, V), two blocks per barrier.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ Dv,
    float* __restrict__ dQ, int BH, int Nq, int Nk, float c, float scale, int n_qt) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[kDqBufs * 2 * T::BYTES];
  lds_char* const lds = (lds_char*)smem;
  auto k_tile = [&](int buf) { return lds + buf * 2 * T::BYTES; };
  auto v_tile = [&](int buf) { return k_tile(buf) + T::BYTES; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int qt = n_qt - 1 - (int)(blockIdx.x / BH), bh = (int)(blockIdx.x % BH);
  const int off = Nk - Nq;
  const int q0w = qt * kFixed + wave * kRows;
  const int q = q0w + col;  // this lane's query
  const bf16* Kh = K + (size_t)bh * Nk * D;
  const bf16* Vh = V + (size_t)bh * Nk * D;

  // Key blocks any query of the workgroup sees (every wave takes all of them).
  const int kv_end = CAUSAL ? min(Nk, min(Nq, (qt + 1) * kFixed) + off) : Nk;
  const int n_kb = kv_end > 0 ? (kv_end + kRows - 1) / kRows : 0;

  bf16x8 qf[T::KS], df[T::KS];
#pragma unroll
  for (int s = 0; s < T::KS; ++s) {
    qf[s] = load_row_op<D>(Q + (size_t)bh * Nq * D, q, Nq, lane, s);
    df[s] = load_row_op<D>(dO + (size_t)bh * Nq * D, q, Nq, lane, s);
  }
  const float l2 = q < Nq ? lse2[(size_t)bh * Nq + q] : __builtin_huge_valf();
  const float dq_row = q < Nq ? Dv[(size_t)bh * Nq + q] : 0.f;
  f32x16 acc[T::NDB];
  zero_acc(acc);
  const OpOffsets<D> oo = op_offsets<D>(lane);

  // K and V blocks go from memory straight into LDS (no staging registers):
  // copy i of a wave fills tile bytes 1024 (wave IPW + i) .. +1023, lane l
  // the 16 bytes of row p / CPR, slot p % CPR (p = 64 (wave IPW + i) + l),
  // so the lane fetches the chunk that slot holds.  Rows past Nk fetch row
  // Nk-1 (finite values whose P is masked to 0).
  constexpr int IPW = T::BYTES / 1024 / kWaves;
  const char* const kg = reinterpret_cast<const char*>(Kh);
  const char* const vg = reinterpret_cast<const char*>(Vh);
  const uint32_t lds_wave = (uint32_t)(size_t)lds + wave * IPW * 1024;
  auto stage = [&](int kb, int buf) {
    uint32_t dst = lds_wave;
    asm volatile("" : "+s"(dst));
    dst += buf * 2 * T::BYTES;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int p = (wave * IPW + i) * 64 + lane;
      const int r = p / T::CPR, slot = p % T::CPR;
      const uint32_t off = (uint32_t)(min(kb * kRows + r, Nk - 1) * T::ROWB + swz<D>(r, slot) * 16);
      copy_to_lds(kg, off, dst + i * 1024);
      copy_to_lds(vg, off, dst + T::BYTES + i * 1024);
    }
  };
  // Four LDS buffers; key block kb uses buffer kb % 4.  Block kb + 2 is
  // copied at the start of block kb, and every second block ends with a
  // wait for all copies and a barrier: block kb writes buffer (kb+2) % 4,
  // last read by block kb-2, and reads buffer kb % 4, whose copies were
  // waited for before the barrier after block kb-1 (kb even) or kb-2 (kb
  // odd); a barrier lies between each pair.
  if (n_kb > 0) {
    stage(0, 0);
    if (n_kb > 1) stage(1, 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  }
  for (int kb = 0; kb < n_kb; ++kb) {
    const int buf = kb & (kDqBufs - 1);
    paranoid_sync();
    if (kb + 2 < n_kb) stage(kb + 2, (kb + 2) & (kDqBufs - 1));
    paranoid_sync();
    {  // blocks past this wave's last visible key are masked whole
      const lds_char* kt_ = k_tile(buf);
      const lds_char* vt = v_tile(buf);
      // S^T = K Q^T and dP^T = V dO^T: lane = query (column), register r =
      // key 8(r/4) + 4 half + r%4 of the block.  The operands of the first
      // half of the k-steps first; those of the second half are read once
      // the first two products have gone out (fewer registers held).
      constexpr int KH = T::KS / 2;
      bf16x8 ka[T::KS], va[T::KS];
#pragma unroll
      for (int s = 0; s < KH; ++s) {
        const uint32_t a = lane_addr(kt_, oo.row[s]);
        ka[s] = row_at(a, 0);
        va[s] = row_at(a, T::BYTES);  // the V tile follows the K tile
      }
      f32x16 S, dP;
      mm_first(S, ka[0], qf[0]);
      mm_first(dP, va[0], df[0]);
      {
        const lds_char* k0 = kt_;
        const lds_char* v0 = vt;
        after_products(k0, v0);
#pragma unroll
        for (int s = KH; s < T::KS; ++s) {
          const uint32_t a = lane_addr(k0, oo.row[s]);
          ka[s] = row_at(a, 0);
          va[s] = row_at(a, T::BYTES);
        }
      }
#pragma unroll
      for (int s = 1; s < T::KS; ++s) {
        mm_next(S, ka[s], qf[s]);
        mm_next(dP, va[s], df[s]);
      }
      // transposed K operands of the block's first 16 keys, read during the wait
      uint32_t ta[T::NDB][2];
      bf16x8 tk[T::NDB];
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) {
        ta[db][0] = lane_addr(kt_, oo.tr[db][0]);
        ta[db][1] = lane_addr(kt_, oo.tr[db][1]);
        tk[db] = tr_at(ta[db], 0);
      }
      pause_scores(S, dP);
      const int k0 = kb * kRows;
      float dS[16];
      // only blocks at the key end or across this wave's diagonal test keys
      // (a uniform branch around vector work only: no product inside)
      auto softmax = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2_hw(S[r] * c - l2);
          if constexpr (decltype(masked)::value) {
            const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key >= Nk || (CAUSAL && key > q + off)) p = 0.f;
          }
          dS[r] = p * (dP[r] - dq_row);
        }
      };
      if (k0 + kRows > Nk || (CAUSAL && k0 + kRows - 1 > q0w + off))
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
      // dQ^T += K^T dS^T over the block's 32 keys.
      bf16x8 sb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) sb[t] = pack_b(dS, t);
      pause_operands(sb);
      // the first 16 keys' products; the last 16 keys' operands are read
      // while the second half of them runs
      constexpr int H1 = T::NDB / 2;
#pragma unroll
      for (int db = 0; db < H1; ++db) mm_acc(acc[db], tk[db], sb[0]);
      after_products(ta);
      bf16x8 uk[T::NDB];
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) uk[db] = tr_at(ta[db], 16 * T::ROWB);
#pragma unroll
      for (int db = H1; db < T::NDB; ++db) mm_acc(acc[db], tk[db], sb[0]);
#pragma unroll
      for (int db = 0; db < T::NDB; ++db) mm_acc(acc[db], uk[db], sb[1]);
    }
    if ((kb & 1) && kb + 1 < n_kb) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
    }
  }

  pause_acc(acc);
  if (q < Nq) {
    float* dQr = dQ + ((size_t)bh * Nq + q) * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        *reinterpret_cast<f32x4*>(dQr + d0) =
            f32x4{acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale, acc[db][4 * g + 2] * scale,
                  acc[db][4 * g + 3] * scale};
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  float* lse2 = a.ws;
  float* Dv = a.ws + (size_t)BH * a.Nq;
  const long long rows = (long long)BH * a.Nq;
  {
    const unsigned grid = (unsigned)((rows + (kThreads / (D / 8)) - 1) / (kThreads / (D / 8)));
    void* args[] = {(void*)&a.o, (void*)&a.dout, (void*)&a.lse, (void*)&lse2, (void*)&Dv,
                    (void*)&rows};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_rows_kernel<D>),
                                         dim3(grid), dim3(kThreads), args, 0, a.stream);
    if (e != hipSuccess) return e;
  }
  {
    const int n_kt = (int)(((long long)a.Nk + kFixed - 1) / kFixed);
    void* args[] = {(void*)&a.q,  (void*)&a.k,  (void*)&a.v,  (void*)&a.dout, (void*)&lse2,
                    (void*)&Dv,   (void*)&a.dk, (void*)&a.dv, (void*)&BH,     (void*)&a.Nq,
                    (void*)&a.Nk, (void*)&c,    (void*)&a.scale};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, CAUSAL>),
                                         dim3((unsigned)(n_kt * BH)), dim3(kThreads), args, 0,
                                         a.stream);
    if (e != hipSuccess) return e;
  }
  const int n_qt = (int)(((long long)a.Nq + kFixed - 1) / kFixed);
  void* args[] = {(void*)&a.q,  (void*)&a.k,  (void*)&a.v,  (void*)&a.dout, (void*)&lse2,
                  (void*)&Dv,   (void*)&a.dq, (void*)&BH,   (void*)&a.Nq,   (void*)&a.Nk,
                  (void*)&c,    (void*)&a.scale, (void*)&n_qt};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<D, CAUSAL>),
                         dim3((unsigned)(n_qt * BH)), dim3(kThreads), args, 0, a.stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

long long bwd_bf16_grid(int B, int H, int N) {
  return (((long long)N + kFixed - 1) / kFixed) * B * H;
}

}  // namespace fa
