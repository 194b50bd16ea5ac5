// Matrix-core rate and clock probe (measurement support, not part of the
// decode path; built as its own library, libmla_probe.so).
//
// Every wave issues iters x 8 independent MFMAs into four accumulators on
// operands read once from `in` (random or zero values: the caller decides),
// and records its shader-clock cycles (s_memtime) and 100 MHz real time
// (s_memrealtime) around the loop.  Cycles per MFMA per wave give the issue
// rate; cycles over real time give the clock the part ran at while every
// wave kept its matrix core busy.  kind 0: v_mfma_f32_32x32x16_f16; kind 1:
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands, unit scales).
//
// C ABI: mla_probe_mfma_clock(kind, grid, iters, in, out, stream) launches
// `grid` workgroups of 4 waves; `in` is a device array of 1024 floats, `out`
// a device array of grid * 4 * 2 uint64 (cycles, real-time ticks per wave).
// Returns a hipError_t value (0 on success); hipErrorInvalidValue for a
// kind other than 0 or 1, grid outside 1 .. 4096 or iters outside 1 .. 1e6.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256, 1) void probe_kernel(const float* __restrict__ in, unsigned long long* __restrict__ out,
                                                       int iters) {
    const int lane = threadIdx.x & 63;
    f16x8 a0, b0, a1, b1;
    i32x8 qa, qb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a0[i] = (_Float16)in[lane * 16 + i];
        b0[i] = (_Float16)in[lane * 16 + 8 + i];
        a1[i] = (_Float16)in[(63 - lane) * 16 + i];
        b1[i] = (_Float16)in[(63 - lane) * 16 + 8 + i];
        const int ca = __builtin_amdgcn_cvt_pk_fp8_f32(in[lane * 16 + i] * 64.f, in[lane * 16 + 15 - i] * 64.f, 0, false);
        const int cb = __builtin_amdgcn_cvt_pk_fp8_f32(in[(63 - lane) * 16 + i] * 64.f, in[lane * 16 + i] * 32.f, 0, false);
        qa[i] = ca | (cb << 16);
        qb[i] = cb | (ca << 16);
    }
    f32x16 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = f32x16{};
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (KIND == 0)
                c[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16((j & 1) ? a1 : a0, (j & 2) ? b1 : b0, c[j & 3], 0, 0, 0);
            else
                c[j & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qb, c[j & 3], 0, 0, 0, 127, 0, 127);
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    // the accumulators are results as far as the compiler knows
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(c[j]));
    if (lane == 0) {
        const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
        out[2 * w] = t1 - t0;
        out[2 * w + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" int mla_probe_mfma_clock(int kind, int grid, int iters, const float* in, unsigned long long* out,
                                    void* stream) {
    if ((kind != 0 && kind != 1) || grid < 1 || grid > 4096 || iters < 1 || iters > 1000000 || !in || !out)
        return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0) hipLaunchKernelGGL(probe_kernel<0>, dim3(grid), dim3(256), 0, s, in, out, iters);
    else hipLaunchKernelGGL(probe_kernel<1>, dim3(grid), dim3(256), 0, s, in, out, iters);
    return (int)hipGetLastError();
}
