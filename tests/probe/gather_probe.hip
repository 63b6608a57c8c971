// Gather-bandwidth probe for the selected-key access pattern (a measured roof,
// not part of the attention library).
//
// Entry e of an index list names a block: it starts at
//   base + (e / heads) * block_stride + (e % heads) * head_stride
// and is `segs` segments of 512 bytes, `seg_stride` bytes apart (one kv head's
// rows of a block of cells in a [cell][kv head][dim] cache).  The list is cut into
// units (a query row and kv head each); a wave takes one unit at a time and reads
// its blocks in order, U at a time (all loads issued before any is used), folding
// them into a checksum, so the only traffic is the gather itself plus one word per
// wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kSegLanes = 32;          // 16-byte lanes per 512-byte segment

template <int U>
__global__ __launch_bounds__(256) void gather_kernel(const char* base, const int32_t* idx, const int32_t* unit_start,
                                                     int n_units, int heads, long long block_stride,
                                                     int head_stride, int segs, int seg_stride, uint32_t* out) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * 256 + threadIdx.x) >> 6;
    const int n_waves = (gridDim.x * 256) >> 6;
    const int tasks = segs * kSegLanes;          // 16-byte loads per block
    uint32_t acc = 0;
    // one unit (a row and kv head of the workload) per wave at a time, its blocks in
    // list order, as the attention kernel visits them
    for (int unit = wave; unit < n_units; unit += n_waves) {
        const int e_end = unit_start[unit + 1];
        for (int i0 = unit_start[unit]; i0 < e_end; i0 += U) {
            uint4 v[U][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u;
                const int e = i < e_end ? idx[i] : -1;
                const char* b = base + static_cast<long long>(e / heads) * block_stride +
                                static_cast<long long>(e % heads) * head_stride;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int t = lane + 64 * j;
                    if (e >= 0 && t < tasks) {
                        const int seg = t / kSegLanes, off = (t % kSegLanes) * 16;
                        v[u][j] = *reinterpret_cast<const uint4*>(b + static_cast<long long>(seg) * seg_stride + off);
                    } else {
                        v[u][j] = uint4{0u, 0u, 0u, 0u};
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc ^= v[u][j].x ^ v[u][j].y ^ v[u][j].z ^ v[u][j].w;
        }
    }
    out[wave] = acc;
}

// Read bandwidth of one level of the memory hierarchy: every wave reads `iters`
// 1 KiB chunks (16 bytes a lane, one load per chunk) of a window of n_chunks KiB,
// each chunk drawn by a per-wave linear congruential sequence, U loads in flight.
// A window that fits a cache level (but not the one above it) measures that level.
template <int U>
__global__ __launch_bounds__(256) void window_read_kernel(const char* base, unsigned chunk_mask, int iters,
                                                          uint32_t* out) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * 256 + threadIdx.x) >> 6;
    uint32_t x = static_cast<uint32_t>(wave) * 2654435761u + 12345u;   // the same in every lane
    uint32_t acc = 0;
    for (int it = 0; it < iters; it += U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x = x * 1664525u + 1013904223u;
            const unsigned c = (x >> 8) & chunk_mask;
            v[u] = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(c) * 1024 + lane * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[wave] = acc;
}

}  // namespace

// Host entry of the window probe: `base` holds n_chunks KiB (a power of two);
// `groups` work-groups of 256 threads, each wave reading `iters` chunks (a multiple
// of 8); `out` holds one word per wave.  Returns 0, -1 for arguments the kernel
// does not take, -2 on a launch error.
extern "C" int window_read_probe(const void* base, int n_chunks, int iters, uint32_t* out, int groups,
                                 void* stream) {
    if (!base || !out || n_chunks < 1 || (n_chunks & (n_chunks - 1)) != 0 || iters < 8 || iters % 8 != 0 ||
        groups < 1)
        return -1;
    hipLaunchKernelGGL(window_read_kernel<8>, dim3(groups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const char*>(base), static_cast<unsigned>(n_chunks - 1), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Host entry: unit u covers idx[unit_start[u] .. unit_start[u + 1]); launches
// `groups` work-groups of 256 threads; `out` holds one word per wave (4 * groups
// words).  segs * 32 must not exceed 128 (two loads per lane).  Returns 0, or -1
// for arguments the kernel does not take, or -2 on a launch error.
extern "C" int gather_probe(const void* base, const int32_t* idx, const int32_t* unit_start, int n_units,
                            int heads, long long block_stride, int head_stride, int segs, int seg_stride,
                            uint32_t* out, int groups, int unroll, void* stream) {
    if (!base || !idx || !unit_start || !out || n_units < 0 || heads < 1 || segs < 1 ||
        segs * kSegLanes > 128 || groups < 1)
        return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const char* b = static_cast<const char*>(base);
    if (unroll == 4)
        hipLaunchKernelGGL(gather_kernel<4>, dim3(groups), dim3(256), 0, st, b, idx, unit_start, n_units, heads,
                           block_stride, head_stride, segs, seg_stride, out);
    else if (unroll == 8)
        hipLaunchKernelGGL(gather_kernel<8>, dim3(groups), dim3(256), 0, st, b, idx, unit_start, n_units, heads,
                           block_stride, head_stride, segs, seg_stride, out);
    else if (unroll == 16)
        hipLaunchKernelGGL(gather_kernel<16>, dim3(groups), dim3(256), 0, st, b, idx, unit_start, n_units, heads,
                           block_stride, head_stride, segs, seg_stride, out);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
