/*
 * fa_probe.h — measurement aids, not part of the attention path.
 *
 * The decode kernels are bound by HBM bandwidth, and the bandwidth a read of
 * a given size can reach on the device (launch, ramp and tail included) is
 * well below the data-sheet peak for small reads.  The first entry point runs a
 * plain streaming-read kernel over a device buffer so that the decode rates
 * can be set beside the empirical ceiling for the same number of bytes.
 */
#ifndef FA_PROBE_H
#define FA_PROBE_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at `src` (device, 16-byte aligned, bytes a positive
 * multiple of 16) with non-temporal 16-byte loads, 256 KB per 256-thread workgroup, eight
 * loads in flight per lane, and keeps nothing: `sink` (device, >= 4 bytes,
 * owned by the caller) is written only if the XOR of the data equals a fixed
 * constant, so the loads cannot be dropped.  Enqueued on `stream`; returns
 * FA_OK (0), FA_ERR_INVALID_ARG (-1) for a null or misaligned pointer or a
 * bad size, or FA_ERR_HIP (-4) if the launch fails.
 */
int fa_probe_read(const void* src, size_t bytes, unsigned* sink, hipStream_t stream);

/*
 * Instruction-issue probe: what one SIMD can overlap.  The prefill kernels'
 * designs rest on how matrix products, vector arithmetic and LDS operand
 * reads share a SIMD, which no data sheet states; this measures it.
 *
 * `grid` workgroups (1..65535) of 8 waves each, one workgroup per CU (the
 * kernel holds 96 KB of LDS), and waves w and w + 4 share a SIMD.  Waves
 * 0-3 run `role_a` for `n_a` operations, waves 4-7 `role_b` for `n_b`
 * (multiples of 8, at most 2^20, positive unless the role is NONE):
 *   FA_PROBE_NONE             nothing;
 *   FA_PROBE_PRODUCTS         v_mfma_f32_32x32x16_bf16, four independent chains;
 *   FA_PROBE_FMA / _EXP       v_fma_f32 / v_exp_f32, eight independent chains;
 *   FA_PROBE_LDS16            16-byte LDS reads (1 KB per wave), eight in flight;
 *   FA_PROBE_LDS_TR8          transposing 8-byte LDS reads (ds_read_b64_tr_b16), eight in flight;
 *   FA_PROBE_PRODUCT_SOFTMAX  products, each followed by an exp, an fma and a bf16 pack;
 *   FA_PROBE_PRODUCT_8FMA     products, each followed by eight fma.
 * `out` (device, 8-byte aligned, grid * 16 int64, owned by the caller)
 * receives for wave w of workgroup g: out[(8g + w) * 2] = shader-clock
 * cycles of its role (s_memtime before and after), out[(8g + w) * 2 + 1] =
 * its HW_ID register (bits 5:4 = SIMD).  Enqueued on `stream`; returns FA_OK,
 * FA_ERR_INVALID_ARG for an argument out of range (before any HIP call), or
 * FA_ERR_HIP if the launch fails.
 */
enum {
  FA_PROBE_NONE = 0,
  FA_PROBE_PRODUCTS = 1,
  FA_PROBE_FMA = 2,
  FA_PROBE_EXP = 3,
  FA_PROBE_LDS16 = 4,
  FA_PROBE_LDS_TR8 = 5,
  FA_PROBE_PRODUCT_SOFTMAX = 6,
  FA_PROBE_PRODUCT_8FMA = 7
};
int fa_probe_issue(int role_a, int role_b, int n_a, int n_b, int grid, long long* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H */
