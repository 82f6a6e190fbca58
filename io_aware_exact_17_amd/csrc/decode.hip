// decode.hip — single-query attention over a packed variable-length KV cache:
// a split-KV partial kernel and a log-sum-exp merge kernel.
//
// With one new query per sequence the score row is 1 x history and there is
// no N x N matrix; the cost is reading the cached keys and values (and, for a
// single request, the launch itself): FlashAttention explainer
// (cztcode.com/2026/5368) §6.  The kernels are therefore bandwidth kernels:
// no matrix cores, 16-byte loads, many loads in flight per lane, and enough
// workgroups to cover every CU even for one sequence.
//
// Each sequence's keys are cut into chunks of `split_keys`.  A workgroup of
// the split kernel streams one (head, chunk, sequence): every key row (d
// bf16 = 256 B at d=128) is read by a group of d/8 lanes, 16 bytes each; the
// q.k dot product is finished with DPP row reductions; each lane group keeps
// the running state (m, l, u) of the explainer's §2 recurrence, updated once
// per batch of keys; the workgroup's lane groups are then merged through LDS
// and one partial state per chunk goes to the workspace.  The merge kernel
// combines a sequence's chunk states with the block-merge rule of explainer
// §3/§7 (m = max, l and u rescaled by exp(m_i - m) and added) and writes
// O = u / l and LSE = m + ln l.  Cache row addresses are 64-bit.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;

template <int D>
struct DecCfg {
  static constexpr int LPR = D / 8;            // lanes per key row (16 B each)
  static constexpr int NRG = kThreads / LPR;   // key rows covered per pass
  static constexpr int U = D == 128 ? 16 : 8;  // keys per lane group per batch
};

template <int D>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (D == 128) return sum_row16(x);
  else return sum_row8(x);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ offsets,
    float* __restrict__ ws_u, float* __restrict__ ws_ml, int H, int split_keys, int n_splits,
    float c) {
  using C = DecCfg<D>;
  // Heads vary fastest across the grid, so the workgroups running together
  // read neighbouring 256-byte head slices of the same token rows.
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int len = seqlens[b];
  const int k_begin = s * split_keys;
  if (k_begin >= len) return;  // chunk past this sequence's end
  const int k_end = min(len, k_begin + split_keys);
  const size_t base = (size_t)offsets[b];

  const int tid = threadIdx.x;
  const int sub = tid % C::LPR;  // which 8 dims of the row this lane reads
  const int rg = tid / C::LPR;   // lane group

  float qv[8];
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(q + ((size_t)b * H + h) * D + sub * 8);
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

  for (int k = k_begin + rg; k < k_end; k += C::NRG * C::U) {
    u32x4 kr[C::U], vr[C::U];
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      const int kk = k + C::NRG * i;
      kr[i] = kk < k_end ? *reinterpret_cast<const u32x4*>(kp + (base + kk) * row_stride)
                         : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      const int kk = k + C::NRG * i;
      vr[i] = kk < k_end ? *reinterpret_cast<const u32x4*>(vp + (base + kk) * row_stride)
                         : u32x4{0, 0, 0, 0};
    }
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
      sc[i] = (k + C::NRG * i < k_end) ? dot * c : kNegInf;
      mx = fmaxf(mx, sc[i]);
    }
    const float m_new = fmaxf(m, mx);  // finite: key k itself is in range
    const float alpha = exp2_hw(m - m_new);
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
  }

  // Merge the lane groups' states (block-merge rule) through LDS.
  __shared__ float sm_m[C::NRG], sm_l[C::NRG];
  __shared__ float sm_u[C::NRG][D + 4];
  if (sub == 0) {
    sm_m[rg] = m;
    sm_l[rg] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_u[rg][sub * 8 + e] = u[e];
  __syncthreads();
  if (tid < D) {
    float M = kNegInf;
    for (int g = 0; g < C::NRG; ++g) M = fmaxf(M, sm_m[g]);
    float L = 0.f, Uacc = 0.f;
    for (int g = 0; g < C::NRG; ++g) {
      const float f = exp2_hw(sm_m[g] - M);  // empty groups (m = -inf) weigh 0
      L = __builtin_fmaf(f, sm_l[g], L);
      Uacc = __builtin_fmaf(f, sm_u[g][tid], Uacc);
    }
    const size_t slot = ((size_t)b * H + h) * n_splits + s;
    ws_u[slot * D + tid] = Uacc;
    if (tid == 0) {
      ws_ml[slot * 2] = M;
      ws_ml[slot * 2 + 1] = L;
    }
  }
}

// One wave per (sequence, head).  The chunk states are read in parallel: each
// lane holds one chunk's (m, l) for the wave-wide maximum and weight, then
// every lane accumulates two output dims over the chunks, taking the chunk
// weights from the lane that computed them.
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

template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ ws_u, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ seqlens, bf16* __restrict__ O, float* __restrict__ LSE, int H,
    int split_keys, int n_splits) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int len = seqlens[b];
  const int n = min(n_splits, len > 0 ? (len + split_keys - 1) / split_keys : 0);
  const size_t slot0 = ((size_t)b * H + h) * n_splits;

  float M = kNegInf;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, ws_ml[(slot0 + s) * 2]);
  M = wave_max(M);
  float Lp = 0.f;
  for (int s = lane; s < n; s += 64)
    Lp = __builtin_fmaf(exp2_hw(ws_ml[(slot0 + s) * 2] - M), ws_ml[(slot0 + s) * 2 + 1], Lp);
  const float L = wave_sum(Lp);

  const int d0 = 2 * lane;
  const bool has_d = d0 < D;
  float U0 = 0.f, U1 = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int s_l = c0 + lane;
    const float f_l = s_l < n ? exp2_hw(ws_ml[(slot0 + s_l) * 2] - M) : 0.f;
    const int cnt = min(64, n - c0);
#pragma unroll 8
    for (int j = 0; j < cnt; ++j) {
      const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f_l), j));
      if (has_d) {
        const f32x2 w = *reinterpret_cast<const f32x2*>(ws_u + (slot0 + c0 + j) * D + d0);
        U0 = __builtin_fmaf(f, w[0], U0);
        U1 = __builtin_fmaf(f, w[1], U1);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t orow = ((size_t)b * H + h) * D;
  if (has_d) *reinterpret_cast<uint32_t*>(O + orow + d0) = pack_bf16x2(U0 * inv, U1 * inv);
  if (lane == 0) LSE[(size_t)b * H + h] = L > 0.f ? (M + log2_hw(L)) * kLn2 : kNegInf;
}

template <int D>
hipError_t launch(const DecodeArgs& a) {
  const float c = a.scale * kLog2e;
  float* ws_u = a.ws;
  float* ws_ml = a.ws + (size_t)a.B * a.H * a.n_splits * D;
  {
    void* args[] = {(void*)&a.q, (void*)&a.kcache, (void*)&a.vcache, (void*)&a.seqlens,
                    (void*)&a.offsets, (void*)&ws_u, (void*)&ws_ml, (void*)&a.H,
                    (void*)&a.split_keys, (void*)&a.n_splits, (void*)&c};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_split_kernel<D>),
                                   dim3((unsigned)a.H, (unsigned)a.n_splits, (unsigned)a.B),
                                   dim3(kThreads), args, 0, a.stream);
    if (e != hipSuccess) return e;
  }
  void* args[] = {(void*)&ws_u, (void*)&ws_ml, (void*)&a.seqlens, (void*)&a.o, (void*)&a.lse,
                  (void*)&a.H, (void*)&a.split_keys, (void*)&a.n_splits};
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_merge_kernel<D>),
                         dim3((unsigned)a.H, (unsigned)a.B), dim3(64), args, 0, a.stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
  return a.d == 128 ? launch<128>(a) : launch<64>(a);
}

}  // namespace fa
