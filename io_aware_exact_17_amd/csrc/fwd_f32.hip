// fwd_f32.hip — exact-attention forward pass in plain fp32 (fp32 in, fp32
// out, fp32 products and sums; no reduced-precision matrix instructions).
//
// Same method as the bf16 kernel (FlashAttention explainer,
// cztcode.com/2026/5368, §2: per-row running max m, sum l and unnormalised
// output u, rescaled whenever m grows; output u / l at the end), written for
// clarity rather than speed: the key/value tile is staged in LDS and every
// query row walks the tile's keys one at a time with the exact per-key update
// of the explainer's recurrence.
//
// Each query row is split over a lane pair (l, l+32): each lane holds half of
// q and half of the output accumulator, the two partial dot products are
// added with one v_permlane32_swap.  4 waves x 32 rows = 128 rows per
// workgroup; causal tiles above the diagonal are not visited.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBR = 128;
constexpr int kBC = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int Nq, int Nk, float c,
    int n_qtiles) {
  constexpr int HD = D / 2;
  __shared__ __attribute__((aligned(16))) float sk[kBC * D];
  __shared__ __attribute__((aligned(16))) float sv[kBC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int q0 = qt * kBR;
  const int off = Nk - Nq;
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;
  const int qi = q0 + wave * 32 + col;
  const int lim = CAUSAL ? min(Nk - 1, qi + off) : Nk - 1;  // last visible key
  const int kv_end = CAUSAL ? min(Nk, q0 + kBR + off) : Nk;

  float q[HD], o[HD];
  {
    const bool ok = qi < Nq;
    const float* src = Q + qbase + (size_t)(ok ? qi : 0) * D + half * HD;
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      q[e] = ok ? src[e] : 0.f;
      o[e] = 0.f;
    }
  }
  float m = kNegInf;  // running max of score * c (log2 units)
  float l = 0.f;

  for (int k0 = 0; k0 < kv_end; k0 += kBC) {
    __syncthreads();
    for (int idx = tid; idx < kBC * D / 4; idx += kThreads) {
      const int key = idx / (D / 4), c4 = idx % (D / 4);
      const int gk = k0 + key;
      f32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (gk < Nk) {
        kv = *reinterpret_cast<const f32x4*>(K + kbase + (size_t)gk * D + c4 * 4);
        vv = *reinterpret_cast<const f32x4*>(V + kbase + (size_t)gk * D + c4 * 4);
      }
      *reinterpret_cast<f32x4*>(sk + key * D + c4 * 4) = kv;
      *reinterpret_cast<f32x4*>(sv + key * D + c4 * 4) = vv;
    }
    __syncthreads();

    const int n = min(kBC, kv_end - k0);
    for (int j = 0; j < n; ++j) {
      const float* kr = sk + j * D + half * HD;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) part = __builtin_fmaf(q[e], kr[e], part);
      float s = sum_across_halves(part) * c;
      if (k0 + j > lim) s = kNegInf;
      if (s > m) {  // the reference moves: rescale l and u by 2^(m_old - m_new)
        const float alpha = exp2_hw(m - s);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < HD; ++e) o[e] *= alpha;
        m = s;
      }
      const float p = (s == kNegInf) ? 0.f : exp2_hw(s - m);
      l += p;
      const float* vr = sv + j * D + half * HD;
#pragma unroll
      for (int e = 0; e < HD; ++e) o[e] = __builtin_fmaf(p, vr[e], o[e]);
    }
  }

  if (qi < Nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = O + qbase + (size_t)qi * D + half * HD;
#pragma unroll
    for (int e = 0; e < HD; e += 4)
      *reinterpret_cast<f32x4*>(dst + e) = f32x4{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
    if (half == 0) LSE[(size_t)bh * Nq + qi] = l > 0.f ? (m + log2_hw(l)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int n_qtiles = (int)(((long long)a.Nq + kBR - 1) / kBR);
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  void* args[] = {(void*)&a.q, (void*)&a.k, (void*)&a.v, (void*)&a.o, (void*)&a.lse,
                  (void*)&BH, (void*)&a.Nq, (void*)&a.Nk, (void*)&c, (void*)&n_qtiles};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_f32_kernel<D, CAUSAL>),
                         dim3((unsigned)(n_qtiles * BH)), dim3(kThreads), args, 0, a.stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

long long fwd_f32_grid(int B, int H, int Nq) {
  return (((long long)Nq + kBR - 1) / kBR) * B * H;
}

}  // namespace fa
