// decode.hip — single-query attention over a packed variable-length KV cache.
//
// With one new query per sequence the score row is 1 x history and there is
// no N x N matrix; the cost is reading the cached keys and values (and, for a
// single request, the launch itself): FlashAttention explainer
// (cztcode.com/2026/5368) §6.  These are bandwidth kernels: no matrix cores,
// 16-byte loads, two batches of loads in flight per lane, enough workgroups
// to cover every CU even for one sequence, and a merge built from parallel
// loads so that it costs a few memory latencies.
//
// Each sequence's keys are cut into chunks of `split_keys`.  A workgroup of
// the split kernel streams one (head, chunk, sequence): every key row (d bf16
// = 256 B at d=128) is read by a group of d/8 lanes, 16 bytes each; the q.k
// dot product is finished with DPP row reductions; each lane group keeps the
// running state (m, l, u) of the explainer's §2 recurrence, updated once per
// batch of keys; the lane groups are merged through LDS with the block-merge
// rule of explainer §3/§7 (m = max, l and u rescaled by exp(m_i - m) and
// added).  A sequence that fits in one chunk is finished on the spot;
// otherwise the chunk's state goes to the workspace and the merge kernel
// combines a sequence's chunk states with the same rule, writing O = u / l
// and LSE = m + ln l.  Cache row addresses are 64-bit.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunkPages = 1024;  // pages one chunk may span (paged cache)

template <int D>
struct DecCfg {
  static constexpr int LPR = D / 8;           // lanes per key row (16 B each)
  static constexpr int NRG = kThreads / LPR;  // key rows covered per pass
  static constexpr int U = 8;                 // keys per lane group per batch
};

template <int D>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (D == 128) return sum_row16(x);
  else return sum_row8(x);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// PAGED: the cache is a pool of pages [num_pages, page_size, H, d] and
// sequence b's key t lives in page block_table[b][t / page_size], slot
// t % page_size (page_size a power of two); otherwise the cache is packed
// and sequence b owns rows offsets[b] ...
template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ block_table, int bt_stride, int page_shift, int num_pages,
    bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ ws_u,
    float* __restrict__ ws_ml, int H, int split_keys, int n_splits, float c) {
  using C = DecCfg<D>;
  // Heads vary fastest across the grid, so the workgroups running together
  // read neighbouring 256-byte head slices of the same token rows.
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int len = seqlens[b];
  const size_t bh = (size_t)b * H + h;
  if (len <= 0) {  // empty history: O = 0, LSE = -inf
    if (s == 0) {
      if (tid < D / 2) *reinterpret_cast<uint32_t*>(O + bh * D + 2 * tid) = 0u;
      if (tid == 0) LSE[bh] = kNegInf;
    }
    return;
  }
  const int k_begin = s * split_keys;
  if (k_begin >= len) return;  // chunk past this sequence's end
  const int k_end = min(len, k_begin + split_keys);
  const int n_active = min(n_splits, (len + split_keys - 1) / split_keys);
  // Cache row of the sequence's key kk.  Paged: the chunk's page numbers are
  // staged in LDS once (entries out of range read the last page instead of
  // faulting), then every key costs an LDS read, a shift and an add.
  __shared__ int sm_page[PAGED ? kMaxChunkPages : 1];
  size_t base = 0;
  int p0 = 0;
  if constexpr (PAGED) {
    p0 = k_begin >> page_shift;
    const int np = ((k_end - 1) >> page_shift) - p0 + 1;
    const int32_t* bt = block_table + (size_t)b * bt_stride + p0;
    for (int i = tid; i < np; i += kThreads)
      sm_page[i] = (int)min((unsigned)bt[i], (unsigned)(num_pages - 1));
    __syncthreads();
  } else {
    base = (size_t)offsets[b];
  }
  const int page_mask = (1 << page_shift) - 1;
  auto row_of = [&](int kk) -> size_t {
    if constexpr (PAGED)
      return ((size_t)sm_page[(kk >> page_shift) - p0] << page_shift) + (size_t)(kk & page_mask);
    else
      return base + (size_t)kk;
  };

  const int sub = tid % C::LPR;  // which 8 dims of the row this lane reads
  const int rg = tid / C::LPR;   // lane group

  float qv[8];
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(q + bh * D + sub * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[2 * i] = bf16_lo(w[i]);
      qv[2 * i + 1] = bf16_hi(w[i]);
    }
  }

  const size_t row_stride = (size_t)H * D;
  const bf16* kp = kc + (size_t)h * D + sub * 8;
  const bf16* vp = vc + (size_t)h * D + sub * 8;

  float m = kNegInf, l = 0.f;
  float u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) u[e] = 0.f;

  // Batch t covers keys k_begin + rg + NRG*(U*t + i), i < U.  Two batches of
  // loads are in flight: the next one is issued before the current one is
  // consumed.  Keys past k_end read the chunk's first key (in range, finite)
  // and are given score -inf.  Every cache byte is read once per call, so the
  // loads carry the non-temporal hint (about 9% more bandwidth than plain
  // loads on both decode workloads).
  constexpr int kStep = C::NRG * C::U;
  u32x4 kA[C::U], vA[C::U], kB[C::U], vB[C::U];
  auto load = [&](u32x4 (&kr)[C::U], u32x4 (&vr)[C::U], int k0) {
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      int kk = k0 + C::NRG * i;
      kk = kk < k_end ? kk : k_begin;
      const size_t row = row_of(kk);
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + row * row_stride));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + row * row_stride));
    }
  };
  auto consume = [&](const u32x4 (&kr)[C::U], const u32x4 (&vr)[C::U], int k0) {
    float sc[C::U];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = __builtin_fmaf(qv[2 * e], bf16_lo(kr[i][e]), part);
        part = __builtin_fmaf(qv[2 * e + 1], bf16_hi(kr[i][e]), part);
      }
      const float dot = row_sum<D>(part);
      sc[i] = (k0 + C::NRG * i < k_end) ? dot * c : kNegInf;
      mx = fmaxf(mx, sc[i]);
    }
    if (mx == kNegInf) return;  // no key of this batch for this lane group
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2_hw(m - m_new);  // 0 while m = -inf
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] *= alpha;
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      const float p = exp2_hw(sc[i] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[2 * e] = __builtin_fmaf(p, bf16_lo(vr[i][e]), u[2 * e]);
        u[2 * e + 1] = __builtin_fmaf(p, bf16_hi(vr[i][e]), u[2 * e + 1]);
      }
    }
    m = m_new;
  };

  const int k_first = k_begin + rg;
  if (k_first < k_end) {
    load(kA, vA, k_first);
    for (int k0 = k_first;; k0 += 2 * kStep) {
      const bool more1 = k0 + kStep < k_end;
      if (more1) load(kB, vB, k0 + kStep);
      consume(kA, vA, k0);
      if (!more1) break;
      const bool more2 = k0 + 2 * kStep < k_end;
      if (more2) load(kA, vA, k0 + 2 * kStep);
      consume(kB, vB, k0 + kStep);
      if (!more2) break;
    }
  }

  // Merge the lane groups' states (block-merge rule) through LDS; wave 0
  // finishes the chunk, each of its lanes owning dims 2*lane and 2*lane+1.
  __shared__ float sm_m[C::NRG], sm_l[C::NRG];
  __shared__ float sm_u[C::NRG][D + 4];
  if (sub == 0) {
    sm_m[rg] = m;
    sm_l[rg] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_u[rg][sub * 8 + e] = u[e];
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  const int d0 = 2 * lane;
  const bool has_d = d0 < D;
  float M = kNegInf, L = 0.f, U0 = 0.f, U1 = 0.f;
  for (int g = 0; g < C::NRG; ++g) M = fmaxf(M, sm_m[g]);
  for (int g = 0; g < C::NRG; ++g) {
    const float f = exp2_hw(sm_m[g] - M);  // empty groups (m = -inf) weigh 0
    L = __builtin_fmaf(f, sm_l[g], L);
    if (has_d) {
      U0 = __builtin_fmaf(f, sm_u[g][d0], U0);
      U1 = __builtin_fmaf(f, sm_u[g][d0 + 1], U1);
    }
  }

  if (n_active == 1) {  // the whole history was this chunk
    const float inv = 1.f / L;
    if (has_d) *reinterpret_cast<uint32_t*>(O + bh * D + d0) = pack_bf16x2(U0 * inv, U1 * inv);
    if (lane == 0) LSE[bh] = (M + log2_hw(L)) * kLn2;
    return;
  }

  // Leave this chunk's state for the merge kernel.
  const size_t slot = bh * n_splits + s;
  if (has_d) *reinterpret_cast<f32x2*>(ws_u + slot * D + d0) = f32x2{U0, U1};
  if (lane == 0) *reinterpret_cast<f32x2*>(ws_ml + slot * 2) = f32x2{M, L};
}

// One 256-thread workgroup per (sequence, head) merges the chunk states.
// Every chunk's (m, l) is requested at once, together with the sequence
// length, and the four waves then split the chunks for the u sums, so the
// merge costs a few memory latencies rather than one per chunk.  Sequences
// that fitted in one chunk were finished by the split kernel.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(
    const float* __restrict__ ws_u, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ seqlens, bf16* __restrict__ O, float* __restrict__ LSE, int H,
    int split_keys, int n_splits) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t bh = (size_t)b * H + h;
  const size_t slot0 = bh * n_splits;
  __shared__ float sm_f[kThreads];
  __shared__ float sm_red[2][4];
  __shared__ float sm_part[4][D];

  const int len = seqlens[b];
  // chunk states requested before the length is known (unused slots are
  // never read as numbers: they are discarded by a select)
  f32x2 ml = {kNegInf, 0.f};
  if (tid < n_splits) ml = *reinterpret_cast<const f32x2*>(ws_ml + (slot0 + tid) * 2);
  const int n = min(n_splits, len > 0 ? (len + split_keys - 1) / split_keys : 0);
  if (n <= 1) return;  // empty or finished by the split kernel
  const bool active = tid < n;
  const float m_t = active ? ml[0] : kNegInf;
  const float wmax = wave_max(m_t);
  if (lane == 0) sm_red[0][wave] = wmax;
  __syncthreads();
  const float Mg = fmaxf(fmaxf(sm_red[0][0], sm_red[0][1]), fmaxf(sm_red[0][2], sm_red[0][3]));
  const float f = active ? exp2_hw(m_t - Mg) : 0.f;
  const float wl = wave_sum(active ? f * ml[1] : 0.f);
  sm_f[tid] = f;
  if (lane == 0) sm_red[1][wave] = wl;
  __syncthreads();

  // wave w sums chunks w, w+4, w+8, ... for dims 2*lane, 2*lane+1
  const int d0 = 2 * lane;
  float G0 = 0.f, G1 = 0.f;
  if (d0 < D) {
#pragma unroll 8
    for (int t = wave; t < n; t += 4) {
      const f32x2 w = *reinterpret_cast<const f32x2*>(ws_u + (slot0 + t) * D + d0);
      G0 = __builtin_fmaf(sm_f[t], w[0], G0);
      G1 = __builtin_fmaf(sm_f[t], w[1], G1);
    }
    sm_part[wave][d0] = G0;
    sm_part[wave][d0 + 1] = G1;
  }
  __syncthreads();
  if (wave == 0) {
    const float Lg = sm_red[1][0] + sm_red[1][1] + sm_red[1][2] + sm_red[1][3];
    const float inv = 1.f / Lg;
    if (d0 < D) {
      const float o0 = sm_part[0][d0] + sm_part[1][d0] + sm_part[2][d0] + sm_part[3][d0];
      const float o1 = sm_part[0][d0 + 1] + sm_part[1][d0 + 1] + sm_part[2][d0 + 1] + sm_part[3][d0 + 1];
      *reinterpret_cast<uint32_t*>(O + bh * D + d0) = pack_bf16x2(o0 * inv, o1 * inv);
    }
    if (lane == 0) LSE[bh] = (Mg + log2_hw(Lg)) * kLn2;
  }
}

template <int D, bool PAGED>
hipError_t launch(const DecodeArgs& a) {
  const float c = a.scale * kLog2e;
  float* ws_u = a.ws;
  float* ws_ml = ws_u + (size_t)a.B * a.H * a.n_splits * D;
  {
    void* args[] = {(void*)&a.q,          (void*)&a.kcache,    (void*)&a.vcache,
                    (void*)&a.seqlens,    (void*)&a.offsets,   (void*)&a.block_table,
                    (void*)&a.bt_stride,  (void*)&a.page_shift, (void*)&a.num_pages,
                    (void*)&a.o,          (void*)&a.lse,       (void*)&ws_u,
                    (void*)&ws_ml,        (void*)&a.H,         (void*)&a.split_keys,
                    (void*)&a.n_splits,   (void*)&c};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void*>(&decode_split_kernel<D, PAGED>),
        dim3((unsigned)a.H, (unsigned)a.n_splits, (unsigned)a.B), dim3(kThreads), args, 0, a.stream);
    if (e != hipSuccess) return e;
  }
  if (a.n_splits == 1) return hipSuccess;  // every sequence finished in the split kernel
  void* args[] = {(void*)&ws_u, (void*)&ws_ml, (void*)&a.seqlens, (void*)&a.o, (void*)&a.lse,
                  (void*)&a.H, (void*)&a.split_keys, (void*)&a.n_splits};
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_merge_kernel<D>),
                         dim3((unsigned)a.H, (unsigned)a.B), dim3(kThreads), args, 0, a.stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.block_table)
    return a.d == 128 ? launch<128, true>(a) : launch<64, true>(a);
  return a.d == 128 ? launch<128, false>(a) : launch<64, false>(a);
}

}  // namespace fa
