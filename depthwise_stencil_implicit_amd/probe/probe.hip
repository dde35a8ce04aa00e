// Ceiling probes for gfx950 (measurement only; not part of the convolution
// library): the issue rate of dense bf16 MFMAs, of the vector unit's packed
// bf16 dot2 and fp32 FMA, and the read bandwidth of LDS, each from a kernel
// that does nothing else.  The benchmark times them
// with events and prints the achieved rate next to the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Every wave issues `iters` rounds of 8 independent bf16 MFMAs (eight
// accumulators, so no MFMA waits on another's result): 16x16x32 when
// `big` is 0, 32x32x16 otherwise.  Each lane writes one float,
// out[blockIdx.x * blockDim.x + threadIdx.x]; the first lane of each
// workgroup also writes the shader-clock and the constant 100 MHz
// real-time counter ticks its loop took, clk[2 * blockIdx.x + {0, 1}].
__global__ __launch_bounds__(256) void probe_mfma_kernel(float *out, uint64_t *clk, int iters, float seed, int big)
{
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
        b[i] = (__bf16)(seed * (float)(blockIdx.x + i));
    }
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    if (!big) {
        // Eight named accumulators: an array of them is rotated through
        // registers by the allocator, which adds moves to every round.
        f32x4 c0_{0.f, 0.f, 0.f, 0.f}, c1_ = c0_, c2_ = c0_, c3_ = c0_, c4_ = c0_, c5_ = c0_, c6_ = c0_, c7_ = c0_;
        for (int it = 0; it < iters; ++it) {
            c0_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0_, 0, 0, 0);
            c1_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1_, 0, 0, 0);
            c2_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2_, 0, 0, 0);
            c3_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3_, 0, 0, 0);
            c4_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4_, 0, 0, 0);
            c5_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5_, 0, 0, 0);
            c6_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6_, 0, 0, 0);
            c7_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7_, 0, 0, 0);
        }
        const f32x4 t = c0_ + c1_ + c2_ + c3_ + c4_ + c5_ + c6_ + c7_;
        s = t[0] + t[1] + t[2] + t[3];
    } else {
        f32x16 c0_, c1_, c2_, c3_;
        for (int e = 0; e < 16; ++e) c0_[e] = 0.f;
        c1_ = c0_;
        c2_ = c0_;
        c3_ = c0_;
        for (int it = 0; it < iters; ++it) {
            c0_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0_, 0, 0, 0);
            c1_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1_, 0, 0, 0);
            c2_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2_, 0, 0, 0);
            c3_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3_, 0, 0, 0);
        }
        const f32x16 t = c0_ + c1_ + c2_ + c3_;
        s = t[0] + t[5] + t[10] + t[15];
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// Every wave issues `iters` rounds of 8 independent vector multiply-adds
// per lane (eight accumulators, so none waits on another's result):
// v_dot2_f32_bf16 (two products per lane) when `kind` is 0, v_fma_f32 (one)
// when it is 1.  Kinds 2-4 issue the accumulating dot2 form with operands in
// fixed registers, to see whether register banks (register number mod 4)
// shared between operands slow the issue: 2 = accumulator and both sources
// in one bank, 3 = three different banks, 4 = accumulator and second source
// in one bank.  Outputs as in probe_mfma_kernel.
__global__ __launch_bounds__(256) void probe_valu_kernel(float *out, uint64_t *clk, int iters, float seed, int kind)
{
    const float fa = seed * (float)(threadIdx.x + 1), fb = seed * (float)(blockIdx.x + 3);
    const bf16x2 a{(__bf16)fa, (__bf16)(fa + 1.f)}, b{(__bf16)fb, (__bf16)(fb + 2.f)};
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float s0 = 0.f, s1 = 1.f, s2 = 2.f, s3 = 3.f, s4 = 4.f, s5 = 5.f, s6 = 6.f, s7 = 7.f;
    if (kind == 0) {
#pragma unroll 4
        for (int it = 0; it < iters; ++it) {
            s0 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s0, false);
            s1 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s1, false);
            s2 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s2, false);
            s3 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s3, false);
            s4 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s4, false);
            s5 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s5, false);
            s6 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s6, false);
            s7 = __builtin_amdgcn_fdot2_f32_bf16(a, b, s7, false);
        }
    } else {
#pragma unroll 4
        for (int it = 0; it < iters; ++it) {
            s0 = __builtin_fmaf(fa, fb, s0);
            s1 = __builtin_fmaf(fa, fb, s1);
            s2 = __builtin_fmaf(fa, fb, s2);
            s3 = __builtin_fmaf(fa, fb, s3);
            s4 = __builtin_fmaf(fa, fb, s4);
            s5 = __builtin_fmaf(fa, fb, s5);
            s6 = __builtin_fmaf(fa, fb, s6);
            s7 = __builtin_fmaf(fa, fb, s7);
        }
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    out[blockIdx.x * blockDim.x + threadIdx.x] = s0 + s1 + s2 + s3 + s4 + s5 + s6 + s7;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// Kinds 2-4 of probe_valu: the accumulating dot2 form with operands in
// fixed registers (one kernel per kind, so that no kind's register choices
// carry over to another's loop as copies).
template <int KIND>
__global__ __launch_bounds__(256) void probe_bank_kernel(float *out, uint64_t *clk, int iters, float seed)
{
    const float fa = seed * (float)(threadIdx.x + 1), fb = seed * (float)(blockIdx.x + 3);
    const bf16x2 a{(__bf16)fa, (__bf16)(fa + 1.f)}, b{(__bf16)fb, (__bf16)(fb + 2.f)};
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    float s0 = 0.f, s1 = 1.f, s2 = 2.f, s3 = 3.f, s4 = 4.f, s5 = 5.f, s6 = 6.f, s7 = 7.f;
    const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
#define PROBE_DOT8(A0, A1, A2, A3, A4, A5, A6, A7, X, Y)                                                          \
    asm volatile("v_dot2c_f32_bf16 %0, %8, %9\n v_dot2c_f32_bf16 %1, %8, %9\n v_dot2c_f32_bf16 %2, %8, %9\n"        \
                 " v_dot2c_f32_bf16 %3, %8, %9\n v_dot2c_f32_bf16 %4, %8, %9\n v_dot2c_f32_bf16 %5, %8, %9\n"       \
                 " v_dot2c_f32_bf16 %6, %8, %9\n v_dot2c_f32_bf16 %7, %8, %9"                                    \
                 : "+{" A0 "}"(s0), "+{" A1 "}"(s1), "+{" A2 "}"(s2), "+{" A3 "}"(s3), "+{" A4 "}"(s4),           \
                   "+{" A5 "}"(s5), "+{" A6 "}"(s6), "+{" A7 "}"(s7)                                              \
                 : "{" X "}"(ua), "{" Y "}"(ub))
    if constexpr (KIND == 2) {
#pragma unroll 4
        for (int it = 0; it < iters; ++it)
            PROBE_DOT8("v40", "v44", "v48", "v52", "v56", "v60", "v64", "v68", "v72", "v76");
    } else if constexpr (KIND == 3) {
#pragma unroll 4
        for (int it = 0; it < iters; ++it)
            PROBE_DOT8("v41", "v45", "v49", "v53", "v57", "v61", "v65", "v69", "v74", "v79");
    } else {
#pragma unroll 4
        for (int it = 0; it < iters; ++it)
            PROBE_DOT8("v40", "v44", "v48", "v52", "v56", "v60", "v64", "v68", "v74", "v76");
    }
#undef PROBE_DOT8
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    out[blockIdx.x * blockDim.x + threadIdx.x] = s0 + s1 + s2 + s3 + s4 + s5 + s6 + s7;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// Every lane reads `iters` 16-byte LDS words (ds_read_b128, consecutive
// lanes on consecutive words, so no bank conflicts) from a 64 KiB buffer it
// first fills, folds them into a register, and writes one word per lane.
__global__ __launch_bounds__(256) void probe_lds_kernel(uint32_t *out, int iters)
{
    __shared__ uint4 buf[4096];   // 64 KiB
    for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = uint4{(uint32_t)i, (uint32_t)i + 1u, 3u, 5u};
    __syncthreads();
    uint4 acc{0u, 0u, 0u, 0u};
    int idx = threadIdx.x;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint4 v = buf[(idx + u * 256) & 4095];
            acc.x ^= v.x;
            acc.y += v.y;
            acc.z ^= v.z;
            acc.w += v.w;
        }
        idx = (idx + 64) & 4095;
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

extern "C" __attribute__((visibility("default"))) int probe_mfma(void *out, void *clk, int blocks, int iters,
                                                                  int big, void *stream)
{
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float *)out,
                       (uint64_t *)clk, iters, 1e-3f, big);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" __attribute__((visibility("default"))) int probe_valu(void *out, void *clk, int blocks, int iters,
                                                                  int kind, void *stream)
{
    if (kind == 2)
        hipLaunchKernelGGL(probe_bank_kernel<2>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float *)out,
                           (uint64_t *)clk, iters, 1e-3f);
    else if (kind == 3)
        hipLaunchKernelGGL(probe_bank_kernel<3>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float *)out,
                           (uint64_t *)clk, iters, 1e-3f);
    else if (kind == 4)
        hipLaunchKernelGGL(probe_bank_kernel<4>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float *)out,
                           (uint64_t *)clk, iters, 1e-3f);
    else
        hipLaunchKernelGGL(probe_valu_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float *)out,
                           (uint64_t *)clk, iters, 1e-3f, kind);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" __attribute__((visibility("default"))) int probe_lds(void *out, int blocks, int iters, void *stream)
{
    hipLaunchKernelGGL(probe_lds_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint32_t *)out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
