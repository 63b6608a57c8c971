// Split-K decode followed by the log-sum-exp combine, with the split partials in a
// scratch array the library holds on each device: an entry point for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  It runs the same kernels as
// sel_attn_decode + sel_attn_split_combine and calls no allocating routine.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = SEL_ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The partials of every call on a device.  In host code this name is a host-side
// stand-in; kernels are only ever given the device address looked up below.
__device__ __align__(256) char scratch[kScratchBytes];

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The current device's copy of `scratch` (looked up once per device, with that
// device current), or null with *err set.
void* device_scratch(hipError_t* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    DeviceScratch& d = g_scratch[dev];
    std::call_once(d.once, [&d]() {
        void* p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess) d.ptr = p;
    });
    *err = d.err;
    return d.ptr;
}

// a * b, or cap + 1 when the product exceeds cap
size_t mul_capped(size_t a, size_t b, size_t cap) {
    if (a == 0 || b == 0) return 0;
    return a > cap / b ? cap + 1 : a * b;
}

}  // namespace

extern "C" int sel_attn_decode_noalloc(const sel_attn_decode_args* a, float* out, const float* sinks,
                                       void* hip_stream) {
    if (!a || !out) return SEL_ATTN_EINVAL;
    if (a->part_o || a->part_ml) return SEL_ATTN_EINVAL;          // the partials are the library's
    if (a->n_stream <= 0 || a->n_row <= 0 || a->n_head_q <= 0 || a->head_dim <= 0 || a->cap <= 0 ||
        a->slice_len <= 0)
        return SEL_ATTN_EINVAL;
    // partials [S][R][Hq][ns][D] then [S][R][Hq][ns][2], ns = ceil(cap / slice_len)
    const int64_t ns = (static_cast<int64_t>(a->cap) + a->slice_len - 1) / a->slice_len;
    size_t units = mul_capped(static_cast<size_t>(a->n_stream), static_cast<size_t>(a->n_row), kScratchBytes);
    units = mul_capped(units, static_cast<size_t>(a->n_head_q), kScratchBytes);
    units = mul_capped(units, static_cast<size_t>(ns), kScratchBytes);
    const size_t per_unit = (static_cast<size_t>(a->head_dim) + 2) * sizeof(float);
    if (mul_capped(units, per_unit, kScratchBytes) > kScratchBytes) return SEL_ATTN_EWORKSPACE;
    const size_t o_bytes = units * static_cast<size_t>(a->head_dim) * sizeof(float);

    sel_attn_decode_args d = *a;
    d.n_slices_max = static_cast<int32_t>(ns);
    sel_attn_combine_args c{};
    c.n_stream = a->n_stream;
    c.n_row = a->n_row;
    c.n_head_q = a->n_head_q;
    c.head_dim = a->head_dim;
    c.n_slices_max = static_cast<int32_t>(ns);
    c.kv_len = a->kv_len;
    c.slice_len = a->slice_len;
    c.cap = a->cap;
    c.out = out;
    c.sinks = sinks;
    // both calls are validated in full (with aligned stand-ins for the partials)
    // before the scratch is looked up, so an invalid call touches no device state
    float* const stand_in = reinterpret_cast<float*>(uintptr_t{256});
    d.part_o = d.part_ml = stand_in;
    c.part_o = c.part_ml = stand_in;
    int s = selattn::validate_decode(&d);
    if (s) return s;
    s = selattn::validate_combine(&c);
    if (s) return s;

    hipError_t err = hipSuccess;
    char* base = static_cast<char*>(device_scratch(&err));
    if (!base) return SEL_ATTN_EHIP;
    d.part_o = reinterpret_cast<float*>(base);
    d.part_ml = reinterpret_cast<float*>(base + o_bytes);      // o_bytes is a multiple of 16
    c.part_o = d.part_o;
    c.part_ml = d.part_ml;
    s = sel_attn_decode(&d, hip_stream);
    if (s) return s;
    return sel_attn_split_combine(&c, hip_stream);
}
