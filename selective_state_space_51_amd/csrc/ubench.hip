// ubench.hip - microbenchmarks of the gfx950 resources the scan's roofline argument uses: the
// issue cost of the VALU instruction forms the scan kernels are built from (fp32 FMA and multiply,
// v_exp_f32, v_rcp_f32, an FMA with a scalar operand, a DPP add, the cross-half-wave swaps), the shader clock while they run,
// and the HBM read and copy streams.  Not part of the scan library: it is built into its own shared
// object (libselscan_ubench.so) and driven by selective_state_space_51_amd/ubench.py.
//
// Each VALU kernel keeps 8 independent accumulators per lane and issues `iters` x 8 instructions of
// one form in one asm block per iteration (every instruction reads a register written 8
// instructions earlier, so no DPP or VALU read-after-write wait applies).  Thread 0 of every
// workgroup stamps s_memtime (shader clock) and s_memrealtime (the 100 MHz constant clock) at its
// start and end, so the host can form the clock the kernel ran at.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

enum Kind {
    K_FMA = 0, K_MUL = 1, K_EXP = 2, K_FMA_SGPR = 3, K_DPP_ADD = 4, K_RCP = 5, K_MIX = 6,
    K_FMA_CHAIN1 = 7,   // 8 FMAs on one accumulator: the dependent-issue latency
    K_FMA_CHAIN2 = 8,   // 8 FMAs alternating over two accumulators
    K_EXP_CHAIN1 = 9,   // 8 exps on one register
    K_MIX_INDEP = 10,   // 8 exps and 40 FMAs on separate registers: no FMA reads an exp result
    K_MIX_NEAR = 11,    // 8 exps and 40 FMAs, each exp result read by the FMA right after it
    K_MIX_INDEP3 = 12,  // 8 exps and 24 FMAs on separate registers (1 : 3)
    K_MIX_INDEP19 = 13, // 2 exps and 38 FMAs on separate registers (1 : 19, the backward's mix)
    K_PERMLANE32 = 14,  // 8 v_permlane32_swap on 4 register pairs
    K_PERMLANE16 = 15,  // 8 v_permlane16_swap on 4 register pairs
    K_NKIND
};

template <int KIND>
__global__ __launch_bounds__(256) void ub_valu(float *out, unsigned long long *stamps, int iters, float s) {
    unsigned long long t0 = 0, r0 = 0;
    if (threadIdx.x == 0) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    float a0 = threadIdx.x * 1e-3f, a1 = a0 + 1e-4f, a2 = a0 + 2e-4f, a3 = a0 + 3e-4f, a4 = a0 + 4e-4f,
          a5 = a0 + 5e-4f, a6 = a0 + 6e-4f, a7 = a0 + 7e-4f;
    const float m = 0.999f, c = 1e-6f;
    for (int i = 0; i < iters; ++i) {
        if constexpr (KIND == K_FMA) {
            asm volatile(
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\tv_fmac_f32 %2, %8, %9\n\tv_fmac_f32 %3, %8, %9\n\t"
                "v_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9\n\tv_fmac_f32 %6, %8, %9\n\tv_fmac_f32 %7, %8, %9"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(m), "v"(c));
        } else if constexpr (KIND == K_MUL) {
            asm volatile(
                "v_mul_f32 %0, %0, %8\n\tv_mul_f32 %1, %1, %8\n\tv_mul_f32 %2, %2, %8\n\tv_mul_f32 %3, %3, %8\n\t"
                "v_mul_f32 %4, %4, %8\n\tv_mul_f32 %5, %5, %8\n\tv_mul_f32 %6, %6, %8\n\tv_mul_f32 %7, %7, %8"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(m));
        } else if constexpr (KIND == K_EXP) {
            asm volatile(
                "v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t"
                "v_exp_f32 %4, %4\n\tv_exp_f32 %5, %5\n\tv_exp_f32 %6, %6\n\tv_exp_f32 %7, %7"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
        } else if constexpr (KIND == K_FMA_SGPR) {
            asm volatile(
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\tv_fmac_f32 %2, %8, %9\n\tv_fmac_f32 %3, %8, %9\n\t"
                "v_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9\n\tv_fmac_f32 %6, %8, %9\n\tv_fmac_f32 %7, %8, %9"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "s"(s), "v"(c));
        } else if constexpr (KIND == K_DPP_ADD) {
            asm volatile(
                "v_add_f32_dpp %0, %0, %8 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                "v_add_f32_dpp %1, %1, %8 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                "v_add_f32_dpp %2, %2, %8 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                "v_add_f32_dpp %3, %3, %8 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                "v_add_f32_dpp %4, %4, %8 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                "v_add_f32_dpp %5, %5, %8 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                "v_add_f32_dpp %6, %6, %8 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                "v_add_f32_dpp %7, %7, %8 row_shr:1 row_mask:0xf bank_mask:0xf"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(c));
        } else if constexpr (KIND == K_RCP) {
            asm volatile(
                "v_rcp_f32 %0, %0\n\tv_rcp_f32 %1, %1\n\tv_rcp_f32 %2, %2\n\tv_rcp_f32 %3, %3\n\t"
                "v_rcp_f32 %4, %4\n\tv_rcp_f32 %5, %5\n\tv_rcp_f32 %6, %6\n\tv_rcp_f32 %7, %7"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
        } else if constexpr (KIND == K_FMA_CHAIN1) {
            asm volatile(
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %0, %8, %9\n\t"
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %0, %8, %9"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(m), "v"(c));
        } else if constexpr (KIND == K_FMA_CHAIN2) {
            asm volatile(
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\tv_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\t"
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\tv_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(m), "v"(c));
        } else if constexpr (KIND == K_EXP_CHAIN1) {
            asm volatile(
                "v_exp_f32 %0, %0\n\tv_exp_f32 %0, %0\n\tv_exp_f32 %0, %0\n\tv_exp_f32 %0, %0\n\t"
                "v_exp_f32 %0, %0\n\tv_exp_f32 %0, %0\n\tv_exp_f32 %0, %0\n\tv_exp_f32 %0, %0"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
        } else if constexpr (KIND == K_MIX_INDEP19) {
            float e0 = a0 * 0.5f, e1 = a1 * 0.5f;
            asm volatile(
                "v_exp_f32 %8, %8\n\t"
                "v_fmac_f32 %0, %10, %11\n\tv_fmac_f32 %1, %10, %11\n\tv_fmac_f32 %2, %10, %11\n\tv_fmac_f32 %3, %10, %11\n\t"
                "v_fmac_f32 %4, %10, %11\n\tv_fmac_f32 %5, %10, %11\n\tv_fmac_f32 %6, %10, %11\n\tv_fmac_f32 %7, %10, %11\n\t"
                "v_fmac_f32 %0, %10, %11\n\tv_fmac_f32 %1, %10, %11\n\tv_fmac_f32 %2, %10, %11\n\tv_fmac_f32 %3, %10, %11\n\t"
                "v_fmac_f32 %4, %10, %11\n\tv_fmac_f32 %5, %10, %11\n\tv_fmac_f32 %6, %10, %11\n\tv_fmac_f32 %7, %10, %11\n\t"
                "v_fmac_f32 %0, %10, %11\n\tv_fmac_f32 %1, %10, %11\n\tv_fmac_f32 %2, %10, %11\n\t"
                "v_exp_f32 %9, %9\n\t"
                "v_fmac_f32 %3, %10, %11\n\tv_fmac_f32 %4, %10, %11\n\tv_fmac_f32 %5, %10, %11\n\tv_fmac_f32 %6, %10, %11\n\t"
                "v_fmac_f32 %7, %10, %11\n\tv_fmac_f32 %0, %10, %11\n\tv_fmac_f32 %1, %10, %11\n\tv_fmac_f32 %2, %10, %11\n\t"
                "v_fmac_f32 %3, %10, %11\n\tv_fmac_f32 %4, %10, %11\n\tv_fmac_f32 %5, %10, %11\n\tv_fmac_f32 %6, %10, %11\n\t"
                "v_fmac_f32 %7, %10, %11\n\tv_fmac_f32 %0, %10, %11\n\tv_fmac_f32 %1, %10, %11\n\tv_fmac_f32 %2, %10, %11\n\t"
                "v_fmac_f32 %3, %10, %11\n\tv_fmac_f32 %4, %10, %11\n\tv_fmac_f32 %5, %10, %11"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(e0), "+v"(e1)
                : "v"(m), "v"(c));
            a0 += e0 + e1;
        } else if constexpr (KIND == K_PERMLANE32 || KIND == K_PERMLANE16) {
            // through the builtins, so the compiler places whatever wait states the swaps need
            uint32_t u[8] = {__float_as_uint(a0), __float_as_uint(a1), __float_as_uint(a2), __float_as_uint(a3),
                             __float_as_uint(a4), __float_as_uint(a5), __float_as_uint(a6), __float_as_uint(a7)};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const auto v = KIND == K_PERMLANE32 ? __builtin_amdgcn_permlane32_swap(u[2 * k], u[2 * k + 1], false, false)
                                                        : __builtin_amdgcn_permlane16_swap(u[2 * k], u[2 * k + 1], false, false);
                    u[2 * k] = v[0];
                    u[2 * k + 1] = v[1];
                }
            }
            a0 = __uint_as_float(u[0]), a1 = __uint_as_float(u[1]), a2 = __uint_as_float(u[2]), a3 = __uint_as_float(u[3]);
            a4 = __uint_as_float(u[4]), a5 = __uint_as_float(u[5]), a6 = __uint_as_float(u[6]), a7 = __uint_as_float(u[7]);
            asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
        } else if constexpr (KIND == K_MIX_INDEP || KIND == K_MIX_NEAR || KIND == K_MIX_INDEP3) {
            // exps on e0..e3; FMAs on a0..a7 (K_MIX_NEAR: the FMA after each exp reads its result)
            float e0 = a0 * 0.5f, e1 = a1 * 0.5f, e2 = a2 * 0.5f, e3 = a3 * 0.5f;
            if constexpr (KIND == K_MIX_INDEP) {
                asm volatile(
                    "v_exp_f32 %8, %8\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\t"
                    "v_exp_f32 %9, %9\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\t"
                    "v_exp_f32 %10, %10\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\t"
                    "v_exp_f32 %11, %11\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\t"
                    "v_exp_f32 %8, %8\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\t"
                    "v_exp_f32 %9, %9\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\t"
                    "v_exp_f32 %10, %10\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\t"
                    "v_exp_f32 %11, %11\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13"
                    : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(e0), "+v"(e1),
                      "+v"(e2), "+v"(e3)
                    : "v"(m), "v"(c));
            } else if constexpr (KIND == K_MIX_NEAR) {
                asm volatile(
                    "v_exp_f32 %8, %8\n\tv_fmac_f32 %0, %8, %13\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\t"
                    "v_exp_f32 %9, %9\n\tv_fmac_f32 %5, %9, %13\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\t"
                    "v_exp_f32 %10, %10\n\tv_fmac_f32 %2, %10, %13\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\t"
                    "v_exp_f32 %11, %11\n\tv_fmac_f32 %7, %11, %13\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\t"
                    "v_exp_f32 %8, %8\n\tv_fmac_f32 %4, %8, %13\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\t"
                    "v_exp_f32 %9, %9\n\tv_fmac_f32 %1, %9, %13\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\t"
                    "v_exp_f32 %10, %10\n\tv_fmac_f32 %6, %10, %13\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\t"
                    "v_exp_f32 %11, %11\n\tv_fmac_f32 %3, %11, %13\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13"
                    : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(e0), "+v"(e1),
                      "+v"(e2), "+v"(e3)
                    : "v"(m), "v"(c));
            } else {
                asm volatile(
                    "v_exp_f32 %8, %8\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\t"
                    "v_exp_f32 %9, %9\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\t"
                    "v_exp_f32 %10, %10\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\t"
                    "v_exp_f32 %11, %11\n\tv_fmac_f32 %1, %12, %13\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\t"
                    "v_exp_f32 %8, %8\n\tv_fmac_f32 %4, %12, %13\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\t"
                    "v_exp_f32 %9, %9\n\tv_fmac_f32 %7, %12, %13\n\tv_fmac_f32 %0, %12, %13\n\tv_fmac_f32 %1, %12, %13\n\t"
                    "v_exp_f32 %10, %10\n\tv_fmac_f32 %2, %12, %13\n\tv_fmac_f32 %3, %12, %13\n\tv_fmac_f32 %4, %12, %13\n\t"
                    "v_exp_f32 %11, %11\n\tv_fmac_f32 %5, %12, %13\n\tv_fmac_f32 %6, %12, %13\n\tv_fmac_f32 %7, %12, %13"
                    : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(e0), "+v"(e1),
                      "+v"(e2), "+v"(e3)
                    : "v"(m), "v"(c));
            }
            a0 += e0 + e1 + e2 + e3;
        } else {
            // the scan's per-element mix: 5 fp32 FMA-class operations and 1 exp per element,
            // 9 elements per block of 54 instructions
            asm volatile(
                "v_mul_f32 %0, %0, %8\n\tv_mul_f32 %1, %1, %8\n\tv_exp_f32 %2, %2\n\tv_fmac_f32 %3, %8, %9\n\t"
                "v_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9\n\t"
                "v_mul_f32 %6, %6, %8\n\tv_mul_f32 %7, %7, %8\n\tv_exp_f32 %0, %0\n\tv_fmac_f32 %1, %8, %9\n\t"
                "v_fmac_f32 %2, %8, %9\n\tv_fmac_f32 %3, %8, %9\n\t"
                "v_mul_f32 %4, %4, %8\n\tv_mul_f32 %5, %5, %8\n\tv_exp_f32 %6, %6\n\tv_fmac_f32 %7, %8, %9\n\t"
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\t"
                "v_mul_f32 %2, %2, %8\n\tv_mul_f32 %3, %3, %8\n\tv_exp_f32 %4, %4\n\tv_fmac_f32 %5, %8, %9\n\t"
                "v_fmac_f32 %6, %8, %9\n\tv_fmac_f32 %7, %8, %9\n\t"
                "v_mul_f32 %0, %0, %8\n\tv_mul_f32 %1, %1, %8\n\tv_exp_f32 %2, %2\n\tv_fmac_f32 %3, %8, %9\n\t"
                "v_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9\n\t"
                "v_mul_f32 %6, %6, %8\n\tv_mul_f32 %7, %7, %8\n\tv_exp_f32 %0, %0\n\tv_fmac_f32 %1, %8, %9\n\t"
                "v_fmac_f32 %2, %8, %9\n\tv_fmac_f32 %3, %8, %9\n\t"
                "v_mul_f32 %4, %4, %8\n\tv_mul_f32 %5, %5, %8\n\tv_exp_f32 %6, %6\n\tv_fmac_f32 %7, %8, %9\n\t"
                "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\t"
                "v_mul_f32 %2, %2, %8\n\tv_mul_f32 %3, %3, %8\n\tv_exp_f32 %4, %4\n\tv_fmac_f32 %5, %8, %9\n\t"
                "v_fmac_f32 %6, %8, %9\n\tv_fmac_f32 %7, %8, %9\n\t"
                "v_mul_f32 %0, %0, %8\n\tv_mul_f32 %1, %1, %8\n\tv_exp_f32 %2, %2\n\tv_fmac_f32 %3, %8, %9\n\t"
                "v_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(m), "v"(c));
        }
    }
    out[blockIdx.x * 256 + threadIdx.x] = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
    if (threadIdx.x == 0) {
        const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        stamps[4 * blockIdx.x] = t0;
        stamps[4 * blockIdx.x + 1] = t1;
        stamps[4 * blockIdx.x + 2] = r0;
        stamps[4 * blockIdx.x + 3] = r1;
    }
}

// Read stream: every 16-byte word of [p, p + n) once, 4 loads in flight per thread; one value per
// thread is written so the loads are kept.
__global__ __launch_bounds__(256) void ub_read(const uint4 *p, int64_t n, uint32_t *out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 v0 = p[i], v1 = p[i + stride], v2 = p[i + 2 * stride], v3 = p[i + 3 * stride];
        acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^
               v3.w;
    }
    for (; i < n; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Copy stream: [src, src + n) to [dst, dst + n) in 16-byte words.
__global__ __launch_bounds__(256) void ub_copy(const uint4 *src, uint4 *dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Launch the VALU kernel of `kind` (enum Kind) on `blocks` workgroups of 256 threads, each lane
// issuing iters x 8 instructions (kind 6: iters x 54; kinds 10 and 11: iters x 48; kind 12:
// iters x 32; kind 13: iters x 40).  out: blocks x 256 floats; stamps: blocks x 4 u64.  Returns
// 0, 1 for a bad argument, 2 if the launch was rejected.
int ub_valu_launch(int kind, int blocks, int iters, float *out, unsigned long long *stamps, void *stream) {
    if (kind < 0 || kind >= K_NKIND || blocks <= 0 || iters < 0 || !out || !stamps) return 1;
    const void *k[] = {(const void *)&ub_valu<K_FMA>,        (const void *)&ub_valu<K_MUL>,
                       (const void *)&ub_valu<K_EXP>,        (const void *)&ub_valu<K_FMA_SGPR>,
                       (const void *)&ub_valu<K_DPP_ADD>,    (const void *)&ub_valu<K_RCP>,
                       (const void *)&ub_valu<K_MIX>,        (const void *)&ub_valu<K_FMA_CHAIN1>,
                       (const void *)&ub_valu<K_FMA_CHAIN2>, (const void *)&ub_valu<K_EXP_CHAIN1>,
                       (const void *)&ub_valu<K_MIX_INDEP>,  (const void *)&ub_valu<K_MIX_NEAR>,
                       (const void *)&ub_valu<K_MIX_INDEP3>, (const void *)&ub_valu<K_MIX_INDEP19>,
                       (const void *)&ub_valu<K_PERMLANE32>, (const void *)&ub_valu<K_PERMLANE16>};
    float s = 1e-6f;
    void *args[] = {&out, &stamps, &iters, &s};
    return hipLaunchKernel(k[kind], dim3(blocks), dim3(256), args, 0, (hipStream_t)stream) == hipSuccess ? 0 : 2;
}

// Read n16 16-byte words from p on `blocks` workgroups; out: blocks x 256 u32.
int ub_read_launch(const void *p, int64_t n16, int blocks, uint32_t *out, void *stream) {
    if (!p || !out || n16 < 0 || blocks <= 0) return 1;
    void *args[] = {&p, &n16, &out};
    return hipLaunchKernel((const void *)&ub_read, dim3(blocks), dim3(256), args, 0, (hipStream_t)stream) == hipSuccess
               ? 0
               : 2;
}

// Copy n16 16-byte words from src to dst on `blocks` workgroups.
int ub_copy_launch(const void *src, void *dst, int64_t n16, int blocks, void *stream) {
    if (!src || !dst || n16 < 0 || blocks <= 0) return 1;
    void *args[] = {&src, &dst, &n16};
    return hipLaunchKernel((const void *)&ub_copy, dim3(blocks), dim3(256), args, 0, (hipStream_t)stream) == hipSuccess
               ? 0
               : 2;
}

}  // extern "C"
