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
// mla_probe_mfma_valu (below) prices VALU instructions issued between MFMAs.
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

// VALU work under a running MFMA: one workgroup, every wave a chain of
// MFMAs on two accumulators (as the decode's two score blocks) with N
// independent v_cvt_scalef32_pk_f16_fp8 after each; cycles per MFMA per
// wave.  KIND 0: the scaled fp8 MFMA, accumulators in arch VGPRs (the
// decode's Q.K^T); KIND 1: the f16 MFMA, accumulators in AGPRs (its P.V).
template <int KIND, int N>
__global__ __launch_bounds__(256, 1) void valu_probe_kernel(const float* __restrict__ in,
                                                            unsigned long long* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    i32x8 qa, qb;
    f16x8 a0, b0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        qa[i] = __builtin_amdgcn_cvt_pk_fp8_f32(in[lane * 16 + i], in[lane * 16 + 15 - i], 0, false);
        qb[i] = __builtin_amdgcn_cvt_pk_fp8_f32(in[(63 - lane) * 16 + i], in[lane * 16 + i], 0, false);
        a0[i] = (_Float16)in[lane * 16 + i];
        b0[i] = (_Float16)in[lane * 16 + 8 + i];
    }
    const uint32_t sc = 0x7F7F7F7Fu;          // unit e8m0 scales
    const float fsc = 1.0f;
    uint32_t src[16], d[2][16];
#pragma unroll
    for (int j = 0; j < 16; ++j) src[j] = __builtin_bit_cast(uint32_t, in[(lane * 16 + j) & 1023]);
    f32x16 c0 = {}, c1 = {};
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if constexpr (KIND == 0) {
                if (m == 0)
                    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,0,0] op_sel_hi:[0,0,0]"
                                 : "+v"(c0) : "v"(qa), "v"(qb), "v"(sc), "v"(sc));
                else
                    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,0,0] op_sel_hi:[0,0,0]"
                                 : "+v"(c1) : "v"(qa), "v"(qb), "v"(sc), "v"(sc));
            } else {
                if (m == 0) asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c0) : "v"(a0), "v"(b0));
                else asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c1) : "v"(a0), "v"(b0));
            }
#pragma unroll
            for (int j = 0; j < N; ++j)
                asm volatile("v_cvt_scalef32_pk_f16_fp8 %0, %1, %2" : "=v"(d[m][j]) : "v"(src[j]), "v"(fsc));
        }
    }
    // a 16-pass result needs 19 wait states before it is read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(d[0][j]), "v"(d[1][j]));
    if (lane == 0) out[threadIdx.x >> 6] = t1 - t0;
}

template <int KIND>
hipError_t launch_valu_probe(int n, int iters, const float* in, unsigned long long* out, hipStream_t s) {
    switch (n) {
        case 0: hipLaunchKernelGGL((valu_probe_kernel<KIND, 0>), dim3(1), dim3(256), 0, s, in, out, iters); break;
        case 4: hipLaunchKernelGGL((valu_probe_kernel<KIND, 4>), dim3(1), dim3(256), 0, s, in, out, iters); break;
        case 8: hipLaunchKernelGGL((valu_probe_kernel<KIND, 8>), dim3(1), dim3(256), 0, s, in, out, iters); break;
        case 12: hipLaunchKernelGGL((valu_probe_kernel<KIND, 12>), dim3(1), dim3(256), 0, s, in, out, iters); break;
        case 16: hipLaunchKernelGGL((valu_probe_kernel<KIND, 16>), dim3(1), dim3(256), 0, s, in, out, iters); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// mla_probe_mfma_valu(kind, n_valu, iters, in, out, stream): one workgroup
// of 4 waves; kind 0 the scaled fp8 MFMA (VGPR accumulators), kind 1 the
// f16 MFMA (AGPR accumulators); n_valu in {0, 4, 8, 12, 16} conversions
// after each MFMA; `in` 1024 device floats, `out` 4 device uint64 (cycles
// per wave for iters x 2 MFMAs).  hipErrorInvalidValue for other arguments.
extern "C" int mla_probe_mfma_valu(int kind, int n_valu, int iters, const float* in, unsigned long long* out,
                                   void* stream) {
    if ((kind != 0 && kind != 1) || iters < 1 || iters > 1000000 || !in || !out) return (int)hipErrorInvalidValue;
    if (n_valu != 0 && n_valu != 4 && n_valu != 8 && n_valu != 12 && n_valu != 16) return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    return (int)(kind == 0 ? launch_valu_probe<0>(n_valu, iters, in, out, s)
                           : launch_valu_probe<1>(n_valu, iters, in, out, s));
}

extern "C" int mla_probe_mfma_clock(int kind, int grid, int iters, const float* in, unsigned long long* out,
                                    void* stream) {
    if ((kind != 0 && kind != 1) || grid < 1 || grid > 4096 || iters < 1 || iters > 1000000 || !in || !out)
        return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0) hipLaunchKernelGGL(probe_kernel<0>, dim3(grid), dim3(256), 0, s, in, out, iters);
    else hipLaunchKernelGGL(probe_kernel<1>, dim3(grid), dim3(256), 0, s, in, out, iters);
    return (int)hipGetLastError();
}
