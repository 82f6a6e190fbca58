// probe.hip — measurement aids, not part of the attention path: a plain
// streaming-read kernel (the empirical HBM read ceiling that the decode rates
// are compared with) and an instruction-issue probe (what one SIMD overlaps).
#include <cstdint>

#include "cdna4.hpp"
#include "fa.h"
#include "fa_probe.h"

namespace {

using fa::u32x4;

constexpr int kThreads = 256;
constexpr int kPerWg16 = 256 * 1024 / 16;  // 16-byte words per workgroup
constexpr int kInFlight = 8;               // loads in flight per lane
// Each byte is read once, so the loads carry the non-temporal hint, as the
// decode kernel's cache reads do.

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                        unsigned* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * kPerWg16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < kPerWg16; i += kThreads * kInFlight) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const size_t idx = base + i + (size_t)k * kThreads;
      v[k] = idx < n16 ? __builtin_nontemporal_load(p + idx) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k];
  }
  if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[0] = acc[2];
}

}  // namespace

extern "C" int fa_probe_read(const void* src, size_t bytes, unsigned* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return FA_ERR_INVALID_ARG;
  const size_t n16 = bytes / 16;
  const size_t grid = (n16 + kPerWg16 - 1) / kPerWg16;
  if (grid > 0x7fffffffull) return FA_ERR_INVALID_ARG;
  const fa::u32x4* p = static_cast<const fa::u32x4*>(src);
  void* args[] = {(void*)&p, (void*)&n16, (void*)&sink};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&read_kernel),
                                       dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ------------------------------------------------------------ issue probe
// One 8-wave workgroup per CU (two waves per SIMD: waves w and w + 4 share
// a SIMD; the SIMD numbers HW_ID reports for waves 0-3 are 0, 2, 1, 3); waves 0-3 run role A, waves 4-7 role B, each a fixed number
// of operations, and every wave records its own shader-clock cycles and
// HW_ID.  Comparing a role alone with two roles side by side shows what one
// SIMD's instruction streams can overlap.

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kIssueThreads = 512;
constexpr int kIssueLdsFloats = 24 * 1024;  // 96 KB: one workgroup per CU

__device__ __forceinline__ unsigned hw_id() {
  unsigned r;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(r));
  return r;
}

// Four independent 32x32x16 bf16 products per group of four.
__device__ __forceinline__ float role_products(int n, float seed, int vec_per_product) {
  fa::bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(i + 1));
    b[i] = (__bf16)(seed - (float)i);
  }
  fa::f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[4] = {seed, seed + 1.f, seed + 2.f, seed + 3.f};
  uint32_t pk = 0u;
  for (int i = 0; i < n; i += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fa::f32x16& c = j == 0 ? c0 : j == 1 ? c1 : j == 2 ? c2 : c3;
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
      if (vec_per_product == 1) {
        // the softmax's share of one product: an exp, an fma, a pack
        asm volatile("v_exp_f32 %0, %0\n\tv_fma_f32 %1, %1, %3, %3\n\tv_cvt_pk_bf16_f32 %2, %0, %1"
                     : "+v"(x[j & 1]), "+v"(x[2 + (j & 1)]), "=v"(pk)
                     : "v"(seed));
      } else if (vec_per_product == 2) {
        asm volatile(
            "v_fma_f32 %0, %0, %2, %2\n\tv_fma_f32 %1, %1, %2, %2\n\tv_fma_f32 %0, %0, %2, %2\n\t"
            "v_fma_f32 %1, %1, %2, %2\n\tv_fma_f32 %0, %0, %2, %2\n\tv_fma_f32 %1, %1, %2, %2\n\t"
            "v_fma_f32 %0, %0, %2, %2\n\tv_fma_f32 %1, %1, %2, %2"
            : "+v"(x[j & 1]), "+v"(x[2 + (j & 1)])
            : "v"(seed));
      }
    }
  }
  float s = x[0] + x[1] + x[2] + x[3] + (float)(pk & 1u);
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  return s;
}

__device__ __forceinline__ float role_valu(int n, float seed, bool exp) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = seed * 0.001f * (float)i;
  for (int i = 0; i < n; i += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (exp)
        asm volatile("v_exp_f32 %0, %0" : "+v"(x[j]));
      else
        asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[j]) : "v"(seed), "v"(0.5f));
    }
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  return s;
}

// LDS operand reads from this wave's 4 KB, eight in flight, waited for in
// the statement that issues them: 16-byte reads (1 KB per wave) or
// transposing 8-byte reads.
__device__ __forceinline__ float role_lds(int n, const lds_char* base, int lane, bool transposing) {
  f4 acc = {};
  const lds_char* p = base + lane * 16;
  const lds_char* q = base + lane * 8;
  for (int i = 0; i < n; i += 8) {
    if (transposing) {
      s16x4 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:512\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:1024\n\tds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:2048\n\tds_read_b64_tr_b16 %5, %8 offset:2560\n\t"
          "ds_read_b64_tr_b16 %6, %8 offset:3072\n\tds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)
          : "v"(q)
          : "memory");
      acc[0] += (float)(v0[0] + v1[0] + v2[0] + v3[0]) + (float)(v4[0] + v5[0] + v6[0] + v7[0]);
    } else {
      f4 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile(
          "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
          "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
          "ds_read_b128 %4, %8\n\tds_read_b128 %5, %8 offset:1024\n\t"
          "ds_read_b128 %6, %8 offset:2048\n\tds_read_b128 %7, %8 offset:3072\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)
          : "v"(p)
          : "memory");
      acc += v0 + v1 + v2 + v3 + v4 + v5 + v6 + v7;
    }
  }
  return acc[0] + acc[1] + acc[2] + acc[3];
}

__device__ __forceinline__ float run_role(int role, int n, float seed, const lds_char* base, int lane) {
  switch (role) {
    case FA_PROBE_PRODUCTS: return role_products(n, seed, 0);
    case FA_PROBE_FMA: return role_valu(n, seed, false);
    case FA_PROBE_EXP: return role_valu(n, seed, true);
    case FA_PROBE_LDS16: return role_lds(n, base, lane, false);
    case FA_PROBE_LDS_TR8: return role_lds(n, base, lane, true);
    case FA_PROBE_PRODUCT_SOFTMAX: return role_products(n, seed, 1);
    case FA_PROBE_PRODUCT_8FMA: return role_products(n, seed, 2);
    default: return 0.f;
  }
}

__global__ __launch_bounds__(kIssueThreads, 1) void issue_kernel(int role_a, int role_b, int n_a, int n_b,
                                                                 long long* __restrict__ out, float seed) {
  __shared__ float lds[kIssueLdsFloats];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kIssueLdsFloats; i += kIssueThreads) lds[i] = seed + (float)(i & 255);
  __syncthreads();
  const lds_char* base = (const lds_char*)lds + wave * 4096;
  const bool a = wave < 4;
  const long long t0 = (long long)__builtin_amdgcn_s_memtime();
  const float r = run_role(a ? role_a : role_b, a ? n_a : n_b, seed + (float)threadIdx.x, base, lane);
  const long long t1 = (long long)__builtin_amdgcn_s_memtime();
  if (lane == 0) {
    out[((size_t)blockIdx.x * 8 + wave) * 2] = t1 - t0;
    out[((size_t)blockIdx.x * 8 + wave) * 2 + 1] = (long long)hw_id();
  }
  if (r == 1234.5f) out[0] = -1;  // keeps the work
}

}  // namespace

extern "C" int fa_probe_issue(int role_a, int role_b, int n_a, int n_b, int grid, long long* out,
                              hipStream_t stream) {
  auto bad_role = [](int r) { return r < FA_PROBE_NONE || r > FA_PROBE_PRODUCT_8FMA; };
  auto bad_n = [](int role, int n) {
    return n < 0 || n > (1 << 20) || n % 8 != 0 || (role != FA_PROBE_NONE && n == 0);
  };
  if (bad_role(role_a) || bad_role(role_b) || bad_n(role_a, n_a) || bad_n(role_b, n_b) || grid < 1 ||
      grid > 65535 || !out || reinterpret_cast<uintptr_t>(out) % 8 != 0)
    return FA_ERR_INVALID_ARG;
  const float seed = 1.001f;
  void* args[] = {(void*)&role_a, (void*)&role_b, (void*)&n_a, (void*)&n_b, (void*)&out, (void*)&seed};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&issue_kernel), dim3((unsigned)grid),
                                       dim3(kIssueThreads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
