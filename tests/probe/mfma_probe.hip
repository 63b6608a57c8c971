// One-wave probes on gfx950: the v_mfma_f32_16x16x32_{bf16,f16} lane layout, and
// the e4m3 byte convert (below).
// Each lane passes its own 8 A values and 8 B values (16-bit bit patterns) and
// gets back its 4 accumulator values; the test checks them against the layout
// the attention kernels assume.  Buffers: a, b [64][8] uint16; d [64][4] float.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(64) probe(const uint16_t* a, const uint16_t* b, float* d, int f16) {
    const int l = threadIdx.x;
    u16x8 av, bv;
    for (int j = 0; j < 8; ++j) { av[j] = a[l * 8 + j]; bv[j] = b[l * 8 + j]; }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (f16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av),
                                                     __builtin_bit_cast(f16x8_t, bv), acc, 0, 0, 0);
    else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                      __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
    for (int i = 0; i < 4; ++i) d[l * 4 + i] = acc[i];
}

extern "C" int mfma_probe(const void* a, const void* b, void* d, int f16, void* stream) {
    hipLaunchKernelGGL(probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
                       static_cast<float*>(d), f16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// e4m3 decoding probe: lane l converts the four bytes of word l with the
// v_cvt_f32_fp8 byte-select forms the kernels use; out [64][4] floats.
__global__ void __launch_bounds__(64) fp8_cvt(const uint32_t* w, float* out) {
    const int l = threadIdx.x;
    const int x = static_cast<int>(w[l]);
    out[l * 4 + 0] = __builtin_amdgcn_cvt_f32_fp8(x, 0);
    out[l * 4 + 1] = __builtin_amdgcn_cvt_f32_fp8(x, 1);
    out[l * 4 + 2] = __builtin_amdgcn_cvt_f32_fp8(x, 2);
    out[l * 4 + 3] = __builtin_amdgcn_cvt_f32_fp8(x, 3);
}

// v_cvt_scalef32_pk_bf16_fp8 with scale 1 (two adjacent e4m3 bytes -> two bf16),
// both halves of each word; 256 lanes, out [256][2] packed pairs.
__global__ void __launch_bounds__(256) fp8_pk_cvt(const uint32_t* w, uint32_t* out) {
    const int l = threadIdx.x;
    const int x = static_cast<int>(w[l]);
    out[l * 2 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
    out[l * 2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
}

extern "C" int fp8_pk_probe(const void* w, void* out, void* stream) {
    hipLaunchKernelGGL(fp8_pk_cvt, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint32_t*>(w), static_cast<uint32_t*>(out));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int fp8_probe(const void* w, void* out, void* stream) {
    hipLaunchKernelGGL(fp8_cvt, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint32_t*>(w), static_cast<float*>(out));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
