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
// Mapping to CDNA4:
//  * 4 waves x 32 query rows = 128 rows per workgroup.  Both products run on
//    the matrix cores as v_mfma_f32_32x32x16_bf16.
//  * The score tile is formed transposed, S^T = K Q^T, so every lane holds one
//    query column: the row max and row sum are in-lane reductions plus one
//    exchange between lane halves (v_permlane32_swap); no reduction crosses
//    waves.  The accumulator registers of S^T, rounded to bf16, are directly
//    the B operand of O^T += V^T P^T, so P never leaves registers.
//  * K tiles are staged row-major in LDS; V tiles are staged transposed
//    (V^T, keys contiguous) with the key order permuted inside each group of
//    16 so that one 16-byte LDS read yields exactly the 8 keys a lane's P
//    registers hold.  Row strides are padded by 16 bytes so that the 16-byte
//    LDS reads of 32 different rows are free of bank conflicts.
//  * LDS is double-buffered: the next tile is fetched from HBM into registers
//    with 16-byte loads while the current one is used, then written to the
//    other buffer; one barrier per tile.
//  * exp is evaluated as 2^x on v_exp_f32 with log2(e) folded into the scale.
//    The reference maximum is only moved when a tile's maximum exceeds it by
//    more than 2^8 (probabilities stay <= 256 before rounding to bf16), which
//    skips most rescales of the output accumulator without changing the
//    mathematics.
//  * Workgroups are issued heaviest query tile first; consecutive workgroup
//    ids walk the heads, so when B*H is a multiple of 8 every tile of a head
//    lands on the same XCD (workgroups are dealt round-robin to the 8 XCDs)
//    and shares its K/V in that XCD's L2.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;          // query rows per workgroup
constexpr float kLazyTau = 8.0f;  // log2 headroom before the reference max moves

template <int D>
struct FwdCfg {
  static constexpr int BC = 8192 / D;   // keys per tile: 64 for d=128, 128 for d=64
  static constexpr int KS = D / 16;     // k-steps of S^T = K Q^T
  static constexpr int NKB = BC / 32;   // 32-key blocks per tile
  static constexpr int NDB = D / 32;    // 32-row blocks of O^T
  static constexpr int KROW = D + 8;    // LDS row stride of K (elements)
  static constexpr int VROW = BC + 8;   // LDS row stride of V^T (elements)
  static constexpr int KTILE = BC * KROW;
  static constexpr int VTILE = D * VROW;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KCHUNKS = BC * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int KGROUPS = BC / 4;                 // 4-key groups of a V tile
  static_assert(KCHUNKS * kThreads * 8 == BC * D, "K tile must split evenly");
  static_assert(KGROUPS * (D / 8) == kThreads, "one 4x8 V block per thread");
};

// Position of key `k` (0..15) inside its group of 16 in the V^T layout:
// the two middle groups of four are swapped, so positions 8h..8h+7 hold keys
// {4h..4h+3, 8+4h..8+4h+3} — the keys accumulator registers 0..7 of lane
// half h cover in the S^T layout.
__device__ __forceinline__ int vt_pos4(int group4) {
  return ((group4 & 1) << 1) | ((group4 >> 1) & 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int Nq, int Nk,
    float c, int negate_q, int n_qtiles) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column of this lane in S^T / O^T
  const int half = lane >> 5;  // which 8-wide k slice / 4-row group this lane holds

  // Heaviest query tile first; heads vary fastest.
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int q0 = qt * kBR;
  const int off = Nk - Nq;  // bottom-right causal alignment
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;

  int kv_end = Nk;
  if (CAUSAL) kv_end = min(Nk, q0 + kBR + off);
  const int n_tiles = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  const int wq0 = q0 + wave * 32;  // first query row of this wave
  const int qi = wq0 + col;        // this lane's query row

  // Q^T operand: lane holds Q[qi][16s + 8*half + 0..7] for every k-step s.
  // Rows past Nq read row Nq-1 (their results are never stored).
  bf16x8 qf[C::KS];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(Q + qbase + (size_t)min(qi, Nq - 1) * D);
    const uint32_t flip = negate_q ? 0x80008000u : 0u;  // exact sign flip for a negative scale
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 w = src[2 * s + half];
      w ^= flip;
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Staging registers for the next tile.
  u32x4 kreg[C::KCHUNKS];
  u32x4 vreg[4];
  const int vkg = tid % C::KGROUPS;  // 4-key group of the V block this thread moves
  const int vdb = tid / C::KGROUPS;  // 8-wide d block

  // Per-lane byte offsets inside a tile (the tile base is uniform, so loads
  // take an SGPR base plus a 32-bit lane offset).  Keys past Nk read row
  // Nk-1 instead: finite values whose scores are masked to -inf, so they
  // carry zero weight.  Only a ragged last tile clamps.
  uint32_t koff[C::KCHUNKS], voff[4];
#pragma unroll
  for (int i = 0; i < C::KCHUNKS; ++i) {
    const int ch = tid + kThreads * i;
    koff[i] = (uint32_t)(((ch / (D / 8)) * D + (ch % (D / 8)) * 8) * 2);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) voff[r] = (uint32_t)(((4 * vkg + r) * D + vdb * 8) * 2);

  auto load_tile = [&](int j) {
    const int k0 = j * BC;
    const char* Kt = reinterpret_cast<const char*>(K + kbase + (size_t)k0 * D);
    const char* Vt = reinterpret_cast<const char*>(V + kbase + (size_t)k0 * D);
    if (k0 + BC <= Nk) {
#pragma unroll
      for (int i = 0; i < C::KCHUNKS; ++i) kreg[i] = *reinterpret_cast<const u32x4*>(Kt + koff[i]);
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[r] = *reinterpret_cast<const u32x4*>(Vt + voff[r]);
    } else {
      const int last = Nk - 1 - k0;
#pragma unroll
      for (int i = 0; i < C::KCHUNKS; ++i) {
        const int ch = tid + kThreads * i;
        const uint32_t o = (uint32_t)((min(ch / (D / 8), last) * D + (ch % (D / 8)) * 8) * 2);
        kreg[i] = *reinterpret_cast<const u32x4*>(Kt + o);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t o = (uint32_t)((min(4 * vkg + r, last) * D + vdb * 8) * 2);
        vreg[r] = *reinterpret_cast<const u32x4*>(Vt + o);
      }
    }
  };

  auto store_tile = [&](int stage) {
    bf16* sk = smem + stage * C::STAGE;
    bf16* sv = sk + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::KCHUNKS; ++i) {
      const int ch = tid + kThreads * i;
      const int key = ch / (D / 8), cc = ch % (D / 8);
      *reinterpret_cast<u32x4*>(sk + key * C::KROW + cc * 8) = kreg[i];
    }
    // 4 keys x 8 dims -> 8 rows of V^T, 4 keys each.
    const int pos = 16 * (vkg >> 2) + 4 * vt_pos4(vkg & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t e01 = __builtin_amdgcn_perm(vreg[1][i], vreg[0][i], 0x05040100u);
      const uint32_t e23 = __builtin_amdgcn_perm(vreg[3][i], vreg[2][i], 0x05040100u);
      const uint32_t o01 = __builtin_amdgcn_perm(vreg[1][i], vreg[0][i], 0x07060302u);
      const uint32_t o23 = __builtin_amdgcn_perm(vreg[3][i], vreg[2][i], 0x07060302u);
      *reinterpret_cast<u32x2*>(sv + (vdb * 8 + 2 * i) * C::VROW + pos) = u32x2{e01, e23};
      *reinterpret_cast<u32x2*>(sv + (vdb * 8 + 2 * i + 1) * C::VROW + pos) = u32x2{o01, o23};
    }
  };

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) oacc[i] = f32x16{};
  float m_ref = kNegInf;  // reference maximum, log2 units (score * c)
  float l_part = 0.f;     // this lane half's share of the row sum

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int stage = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    const int k0 = j * BC;
    const bool wave_active = !CAUSAL || k0 <= wq0 + 31 + off;
    if (wave_active) {
      const bf16* sk = smem + stage * C::STAGE;
      const bf16* sv = sk + C::KTILE;

      // S^T = K Q^T for this tile: NKB blocks of 32 keys x 32 queries.
      // The NKB accumulators are independent; alternating them keeps
      // consecutive matrix instructions free of dependences.
      f32x16 sacc[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sk + (kb * 32 + col) * C::KROW + s * 16 + half * 8);
          sacc[kb] = mfma_32x32x16(a, qf[s], sacc[kb]);
        }

      // Mask keys past the end and, on diagonal tiles, keys after the query.
      const bool need_mask = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > wq0 + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(Nk - 1, qi + off) : Nk - 1;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key > lim) sacc[kb][r] = kNegInf;
          }
      }

      // Row maximum of this tile (in-lane, then across the lane halves).
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_across_halves(mx);
      const float mt = mx * c;  // c > 0, so -inf stays -inf

      // Move the reference only when the tile max exceeds it by > 2^tau.
      const bool grow = mt > m_ref + kLazyTau;
      if (wave_any(grow)) {
        const float m_new = grow ? mt : m_ref;
        const float alpha = grow ? exp2_hw(m_ref - m_new) : 1.f;  // 0 when m_ref was -inf
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < C::NDB; ++i) oacc[i] *= alpha;
        m_ref = m_new;
      }
      const float m_use = (m_ref == kNegInf) ? 0.f : m_ref;

      // P = 2^(s*c - m), its row sum, and bf16 pairs for the P^T operand.
      uint32_t pk[C::NKB][8];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = exp2_hw(__builtin_fmaf(sacc[kb][r], c, -m_use));
          const float p1 = exp2_hw(__builtin_fmaf(sacc[kb][r + 1], c, -m_use));
          lsum += p0 + p1;
          pk[kb][r >> 1] = pack_bf16x2(p0, p1);
        }
      l_part += lsum;

      // O^T += V^T P^T over the tile's keys, 16 keys per step.
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 pw = {pk[kb][4 * t], pk[kb][4 * t + 1], pk[kb][4 * t + 2], pk[kb][4 * t + 3]};
          const bf16x8 b = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sv + (db * 32 + col) * C::VROW + (2 * kb + t) * 16 + half * 8);
            oacc[db] = mfma_32x32x16(a, b, oacc[db]);
          }
        }
    }

    if (j + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: one division per row, O in bf16, LSE = ln2 * (m + log2 l).
  const float l_tot = sum_across_halves(l_part);
  if (qi < Nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* orow = O + qbase + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                         pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * g + 4 * half) = w;
      }
    if (half == 0)
      LSE[(size_t)bh * Nq + qi] = l_tot > 0.f ? (m_ref + log2_hw(l_tot)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int n_qtiles = (a.Nq + kBR - 1) / kBR;
  const int BH = a.B * a.H;
  // c > 0 keeps masked scores (-inf) at -inf after scaling.  A zero scale
  // becomes 1e-30: every product with a finite score then rounds away
  // against the reference, so the weights are exactly uniform, as for 0.
  const float c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  const int neg = a.scale < 0.f ? 1 : 0;
  const dim3 grid((unsigned)(n_qtiles * BH));
  const dim3 block(kThreads);
  void* args[] = {(void*)&a.q, (void*)&a.k, (void*)&a.v, (void*)&a.o, (void*)&a.lse,
                  (void*)&BH, (void*)&a.Nq, (void*)&a.Nk, (void*)&c, (void*)&neg,
                  (void*)&n_qtiles};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, CAUSAL>), grid, block,
                         args, 0, a.stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

long long fwd_bf16_grid(int B, int H, int Nq) {
  return (long long)((Nq + kBR - 1) / kBR) * B * H;
}

}  // namespace fa
