// One-wave probes on gfx950: the v_mfma_f32_16x16x32_{bf16,f16} and
// v_mfma_f32_32x32x16_bf16 lane layouts, and the e4m3 byte convert (below).
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

// v_mfma_f32_32x32x16_bf16: 8 A and 8 B values per lane in, 16 accumulator values
// per lane out (d [64][16] float).
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ void __launch_bounds__(64) probe32(const uint16_t* a, const uint16_t* b, float* d) {
    const int l = threadIdx.x;
    u16x8 av, bv;
    for (int j = 0; j < 8; ++j) { av[j] = a[l * 8 + j]; bv[j] = b[l * 8 + j]; }
    f32x16 acc;
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
    for (int i = 0; i < 16; ++i) d[l * 16 + i] = acc[i];
}

extern "C" int mfma32_probe(const void* a, const void* b, void* d, void* stream) {
    hipLaunchKernelGGL(probe32, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), static_cast<float*>(d));
    return hipGetLastError() == hipSuccess ? 0 : -1;
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

// Buffer range checking: a raw (stride 0) descriptor of num_records bytes over the
// start of a larger, fully allocated buffer `src` (at least 4 * 256 bytes), read
// with the same total offset carried either by the VGPR operand or by the SGPR
// operand.  Lane l reads offset 4 l: out[l] through voffset, out[64 + l] through
// soffset (voffset 0).  Every address lies inside `src`, whatever the check does.
__global__ void __launch_bounds__(64) buffer_range(const uint32_t* src, uint32_t* out, int num_records) {
    const int l = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(src), static_cast<short>(0), num_records, 0x00020000);
    out[l] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * l, 0, 0);
    // soffset must be uniform: lane l's value comes from a loop over the 64 offsets
    uint32_t v = 0;
    for (int i = 0; i < 64; ++i) {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(rs, 0, 4 * i, 0);
        if (i == l) v = w;
    }
    out[64 + l] = v;
}

extern "C" int buffer_range_probe(const void* src, void* out, int num_records, void* stream) {
    if (num_records < 0 || num_records > 256) return -1;
    hipLaunchKernelGGL(buffer_range, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(out), num_records);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Buffer loads straight into LDS (buffer_load_dwordx4 ... lds): wave w's lanes
// read 16 bytes each from src at offset 16 * perm(l), perm(l) = 63 - l, and the
// load deposits them in LDS at base + 1 KiB w; the LDS contents are then copied
// out as they lie.  src >= 4 KiB, out [256][4] uint32 (4 waves).
__global__ void __launch_bounds__(256) lds_dma(const uint32_t* src, uint32_t* out) {
    extern __shared__ __align__(16) char lds[];
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(src), static_cast<short>(0), 4096, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(lds + 1024 * w), 16,
        1024 * w + 16 * (63 - l), 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint4 v = reinterpret_cast<const uint4*>(lds)[threadIdx.x];
    out[threadIdx.x * 4 + 0] = v.x;
    out[threadIdx.x * 4 + 1] = v.y;
    out[threadIdx.x * 4 + 2] = v.z;
    out[threadIdx.x * 4 + 3] = v.w;
}

extern "C" int lds_dma_probe(const void* src, void* out, void* stream) {
    hipLaunchKernelGGL(lds_dma, dim3(1), dim3(256), 4096, static_cast<hipStream_t>(stream),
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(out));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// v_permlane32_swap_b32 and v_permlane16_swap_b32 with both operands holding the
// same value x: lane l writes the two results of each (out [64][4]: the 32-lane
// swap's pair, then the 16-lane swap's pair).  The kernels rely on each pair being
// {x[l], x[l ^ 32]} (resp. {x[l], x[l ^ 16]}) in some order.
__global__ void __launch_bounds__(64) permlane_swap(const uint32_t* in, uint32_t* out) {
    const int l = threadIdx.x;
    const uint32_t x = in[l];
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const auto q = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    out[l * 4 + 0] = r[0];
    out[l * 4 + 1] = r[1];
    out[l * 4 + 2] = q[0];
    out[l * 4 + 3] = q[1];
}

extern "C" int permlane_probe(const void* in, void* out, void* stream) {
    hipLaunchKernelGGL(permlane_swap, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint32_t*>(in), static_cast<uint32_t*>(out));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Matrix-core issue rate: `groups` work-groups of four waves (one per SIMD), each
// wave running `iters` rounds of C independent accumulator chains of one product
// shape (16: v_mfma_f32_16x16x32_bf16, 32: v_mfma_f32_32x32x16_bf16).  Wave 0 of
// each work-group writes the s_memtime ticks of its loop to ticks[group] (core clock
// cycles); every lane writes a sum of its accumulators to out[group * 256 + lane] so
// the products are not removed.  Buffers: out [groups][256] float, ticks [groups].
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int SHAPE, int C>
__global__ void __launch_bounds__(256, 1) mfma_rate(float* out, long long* ticks, int iters) {
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(0.001f * static_cast<float>((threadIdx.x + i) & 15));
        b[i] = static_cast<__bf16>(0.002f * static_cast<float>(i));
    }
    f32x4 c[C];
    f32x16 d[C];
    for (int j = 0; j < C; ++j) {
        c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int e = 0; e < 16; ++e) d[j][e] = 0.f;
    }
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < C; ++j) {
            if constexpr (SHAPE == 16) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
            else d[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d[j], 0, 0, 0);
        }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.f;
    for (int j = 0; j < C; ++j) {
        for (int e = 0; e < 4; ++e) s += c[j][e];
        for (int e = 0; e < 16; ++e) s += d[j][e];
    }
    out[blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0) ticks[blockIdx.x] = t1 - t0;
}

extern "C" int mfma_rate_probe(int shape, int chains, int iters, int groups, void* out, void* ticks, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* o = static_cast<float*>(out);
    long long* t = static_cast<long long*>(ticks);
    if (groups <= 0 || iters <= 0) return -1;
    if (shape == 16 && chains == 1) hipLaunchKernelGGL((mfma_rate<16, 1>), dim3(groups), dim3(256), 0, st, o, t, iters);
    else if (shape == 16 && chains == 4) hipLaunchKernelGGL((mfma_rate<16, 4>), dim3(groups), dim3(256), 0, st, o, t, iters);
    else if (shape == 32 && chains == 1) hipLaunchKernelGGL((mfma_rate<32, 1>), dim3(groups), dim3(256), 0, st, o, t, iters);
    else if (shape == 32 && chains == 4) hipLaunchKernelGGL((mfma_rate<32, 4>), dim3(groups), dim3(256), 0, st, o, t, iters);
    else return -1;
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
