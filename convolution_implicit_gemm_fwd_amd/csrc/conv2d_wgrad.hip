// conv2d_wgrad.hip -- launchers of the weight-backward kernels
// (igemm_wgrad.hpp).  A translation unit of its own so that it can be
// compiled with the MFMA accumulators in VGPRs (-mllvm
// -amdgpu-mfma-vgpr-form): in this kernel's loop the default form left
// 76 register copies between AGPRs and VGPRs per step.
#include "convimg.h"
// igemm_common.hpp defines the split-K counter fill kernel, which the other
// unit launches; this unit's copy takes another name so the two do not clash
#define fill_zero_i32 fill_zero_i32_unused_in_wgrad_unit
#include "igemm_pipe.hpp"
#undef fill_zero_i32
#define CONVIMG_WGRAD_KERNELS
#include "igemm_wgrad.hpp"

namespace convimg {

void wgrad_set_attributes()
{
    for (const void *f : {(const void *)igemm_wgrad_bf16<true, true, kWgPF>,
                          (const void *)igemm_wgrad_bf16<true, false, kWgPF>,
                          (const void *)igemm_wgrad_bf16<false, true, kWgPF>,
                          (const void *)igemm_wgrad_bf16<false, false, kWgPF>})
        (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kWgLdsBytes);
}

hipError_t wgrad_launch(const WgArgs &a, bool vx, bool vdy, int grid, hipStream_t stream)
{
    void (*k)(WgArgs) = vx ? (vdy ? igemm_wgrad_bf16<true, true, kWgPF> : igemm_wgrad_bf16<true, false, kWgPF>)
                           : (vdy ? igemm_wgrad_bf16<false, true, kWgPF> : igemm_wgrad_bf16<false, false, kWgPF>);
    hipLaunchKernelGGL(k, dim3(grid), dim3(kWgThreads), kWgLdsBytes, stream, a);
    return hipGetLastError();
}

hipError_t wgrad_tr_launch(const WgArgs &a, int grid, int stages, hipStream_t stream)
{
    if (stages == kWtStagesPair)
        hipLaunchKernelGGL(igemm_wgrad_tr_bf16<kWtStagesPair>, dim3(grid), dim3(kWgThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(igemm_wgrad_tr_bf16<kWtStagesDeep>, dim3(grid), dim3(kWgThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t wgrad_row_launch(const WgArgs &a, int grid, int xi, int stages, hipStream_t stream)
{
    // SEG: units are segments of rows wider than 64 (else whole rows)
    const bool seg = a.rnseg > 1;
    void (*k)(WgArgs) = xi == 24 ? (seg ? igemm_wgrad_row_bf16<24, 3, true> : igemm_wgrad_row_bf16<24, 3, false>)
                      : stages == 3 ? (seg ? igemm_wgrad_row_bf16<16, 3, true> : igemm_wgrad_row_bf16<16, 3, false>)
                                    : (seg ? igemm_wgrad_row_bf16<16, 4, true> : igemm_wgrad_row_bf16<16, 4, false>);
    hipLaunchKernelGGL(k, dim3(grid), dim3(kWrThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t wgrad_f32_launch(const WgArgs &a, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL(igemm_wgrad_f32, dim3(grid), dim3(kWgThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t wgrad_reduce_launch(const float *part, float *dw, int n, int splits, int vec, int lg,
                               hipStream_t stream)
{
    static_assert(kWgRedMaxGroups == 32, "one instantiation a group count");
    void (*const k[])(const float *, float *, int, int, int) = {wgrad_reduce<0>, wgrad_reduce<1>, wgrad_reduce<2>,
                                                                 wgrad_reduce<3>, wgrad_reduce<4>, wgrad_reduce<5>};
    if (lg < 0 || lg > 5)
        return hipErrorInvalidValue;
    const long long cols = kWgReduceThreads >> lg;
    const int blocks = (int)(((long long)n + 4 * cols - 1) / (4 * cols));
    hipLaunchKernelGGL(k[lg], dim3(blocks), dim3(kWgReduceThreads), 0, stream, part, dw, n, splits, vec);
    return hipGetLastError();
}

}  // namespace convimg
