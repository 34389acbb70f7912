// Stale refresh: this step's fresh slice of a map becomes the stale context
// that the next denoising step reads (DistriFusion reuses the previous step's
// activations of the other patches: "DistriFusion：高分辨率扩散模型的分布式并
// 行推理", README mirror, section 概述, figure (c)).
//
//   stale[b, i*h + r, :] = fresh[b, r, :]      r in [0, h)
//
// Per image the destination rows are one contiguous byte range, so the copy
// is B contiguous ranges.  HBM-bound: each byte is read once and written
// once.  16-byte vectors with non-temporal hints (the data is not re-read by
// this kernel), UNROLL independent vectors in flight per thread, and a
// grid-stride loop so any size is covered by a bounded grid.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <typename U>
__global__ __launch_bounds__(kThreads) void refresh_kernel(const U* __restrict__ fresh,
                                                          U* __restrict__ stale,
                                                          int64_t units_per_image,
                                                          int64_t src_stride, int64_t dst_stride,
                                                          int64_t dst_offset) {
    const int64_t b = blockIdx.y;
    const U* src = fresh + b * src_stride;
    U* dst = stale + b * dst_stride + dst_offset;
    const int64_t step = int64_t(gridDim.x) * kThreads * kUnroll;
    for (int64_t base = int64_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x;
         base < units_per_image; base += step) {
        U v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t idx = base + int64_t(u) * kThreads;
            if (idx < units_per_image) v[u] = __builtin_nontemporal_load(src + idx);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t idx = base + int64_t(u) * kThreads;
            if (idx < units_per_image) __builtin_nontemporal_store(v[u], dst + idx);
        }
    }
}

template <typename U>
hipError_t launch_units(const Geom& g, int64_t row_bytes, const void* fresh, void* stale,
                        hipStream_t s) {
    const int64_t h = g.h();
    const int64_t row_units = row_bytes / int64_t(sizeof(U));
    const int64_t units = h * row_units;
    int64_t blocks = ceil_div(units, int64_t(kThreads) * kUnroll);
    const int64_t cap = 4096;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    dim3 grid(unsigned(blocks), unsigned(g.B));
    hipLaunchKernelGGL(refresh_kernel<U>, grid, dim3(kThreads), 0, s,
                       static_cast<const U*>(fresh), static_cast<U*>(stale), units, units,
                       g.H * row_units, g.i * h * row_units);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_refresh(const Geom& g, int64_t row_elems, int elem_bytes, const void* fresh,
                          void* stale, hipStream_t s) {
    const int64_t row_bytes = row_elems * elem_bytes;
    const uintptr_t a = uintptr_t(fresh) | uintptr_t(stale);
    if (row_bytes % 16 == 0 && a % 16 == 0)
        return launch_units<u32x4>(g, row_bytes, fresh, stale, s);
    if (row_bytes % 4 == 0 && a % 4 == 0)
        return launch_units<uint32_t>(g, row_bytes, fresh, stale, s);
    return launch_units<uint16_t>(g, row_bytes, fresh, stale, s);
}

}  // namespace dp
