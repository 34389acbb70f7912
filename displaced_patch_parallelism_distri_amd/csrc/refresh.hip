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
hipError_t launch_units(int64_t B, int64_t rows, int64_t n, int64_t i, int64_t row_bytes,
                        const void* fresh, void* stale, hipStream_t s) {
    const int64_t row_units = row_bytes / int64_t(sizeof(U));
    const int64_t units = rows * row_units;
    int64_t blocks = ceil_div(units, int64_t(kThreads) * kUnroll);
    const int64_t cap = 4096;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(B));
    hipLaunchKernelGGL(refresh_kernel<U>, grid, dim3(kThreads), 0, s,
                       static_cast<const U*>(fresh), static_cast<U*>(stale), units, units,
                       n * rows * row_units, i * rows * row_units);
    return hipGetLastError();
}

hipError_t launch_one(int64_t B, int64_t rows, int64_t n, int64_t i, int64_t row_bytes,
                      const void* fresh, void* stale, hipStream_t s) {
    const uintptr_t a = uintptr_t(fresh) | uintptr_t(stale);
    if (row_bytes % 16 == 0 && a % 16 == 0)
        return launch_units<u32x4>(B, rows, n, i, row_bytes, fresh, stale, s);
    if (row_bytes % 4 == 0 && a % 4 == 0)
        return launch_units<uint32_t>(B, rows, n, i, row_bytes, fresh, stale, s);
    return launch_units<uint16_t>(B, rows, n, i, row_bytes, fresh, stale, s);
}

// ---------------------------------------------------------------------------
// All of a layer's maps in one launch.  The work is cut into chunks of
// kChunk 16-byte units (128 KiB), each inside one (map, image) range: map m's
// images take chunks [chunk_start_m, chunk_start_m + B * chunks_per_image_m)
// of one index space.  A block copies one chunk at a time (each thread
// kMapUnroll loads in flight, then the stores) and strides over the chunks;
// the grid is one block per CU.  (Measured on MI355X over the SDXL 3840
// layers' maps, 55 and 28 MB per call: 256-1024 threads, 4-16 vectors per
// thread and 1-4 blocks per CU all land within 8% of each other; this shape
// was the fastest, at about 5.4 and 4.65 TB/s.)  A chunk's source
// and destination are buffer resources ending with the chunk's last unit, so
// the tail of a range needs no branch: loads past it return zeros and
// stores past it are dropped.
constexpr int kMapThreads = 512;
constexpr int kMapUnroll = 16;
constexpr int64_t kChunk = int64_t(kMapThreads) * kMapUnroll;
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource, gfx9 family
constexpr int kNontemporal = 2;            // cache-policy bit: no reuse expected

struct MapDesc {
    const u32x4* fresh;
    u32x4* stale;
    int64_t units;        // 16-byte units of one image's fresh slice
    int64_t dst_stride;   // units between images in stale
    int64_t dst_offset;   // units from an image's start to patch i's rows
    int64_t chunk_start;  // first chunk of this map
    int64_t chunks_per_image;
};
struct MapsArgs {
    MapDesc m[kRefreshMaxMaps];
    int count;
    int64_t total_chunks;
};

__global__ __launch_bounds__(kMapThreads) void refresh_maps_kernel(MapsArgs a) {
    const int tid = threadIdx.x;
    for (int64_t c = blockIdx.x; c < a.total_chunks; c += gridDim.x) {
        int m = 0;
        for (int j = 1; j < a.count; ++j)
            if (c >= a.m[j].chunk_start) m = j;
        const MapDesc& d = a.m[m];
        const int64_t rel = c - d.chunk_start;
        const int64_t img = rel / d.chunks_per_image;
        const int64_t u0 = (rel - img * d.chunks_per_image) * kChunk;
        const int64_t left = d.units - u0;
        const int nrec = int((left < kChunk ? left : kChunk) * 16);
        const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<u32x4*>(d.fresh + img * d.units + u0), 0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
            d.stale + img * d.dst_stride + d.dst_offset + u0, 0, nrec, kBufferFlags);
        u32x4 v[kMapUnroll];
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(src, (tid + u * kMapThreads) * 16, 0,
                                                         kNontemporal);
#pragma unroll
        for (int u = 0; u < kMapUnroll; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(v[u], dst, (tid + u * kMapThreads) * 16, 0,
                                                   kNontemporal);
    }
}

}  // namespace

hipError_t launch_refresh(const Geom& g, int64_t row_elems, int elem_bytes, const void* fresh,
                          void* stale, hipStream_t s) {
    return launch_one(g.B, g.h(), g.n, g.i, row_elems * elem_bytes, fresh, stale, s);
}

hipError_t launch_refresh_maps(const Geom& g, int count, const RefreshMap* maps, hipStream_t s) {
    MapsArgs a{};
    int64_t chunks = 0;
    for (int k = 0; k < count; ++k) {
        const RefreshMap& r = maps[k];
        const int64_t row_bytes = r.row_elems * r.elem_bytes;
        const int64_t bytes = r.rows * row_bytes;
        if (bytes == 0 || g.B == 0) continue;
        const uintptr_t al = uintptr_t(r.fresh) | uintptr_t(r.stale);
        if (row_bytes % 16 != 0 || al % 16 != 0) {
            // not whole 16-byte vectors: a launch of its own
            const hipError_t e = launch_one(g.B, r.rows, g.n, g.i, row_bytes, r.fresh, r.stale, s);
            if (e != hipSuccess) return e;
            continue;
        }
        MapDesc& d = a.m[a.count++];
        d.fresh = static_cast<const u32x4*>(r.fresh);
        d.stale = static_cast<u32x4*>(r.stale);
        d.units = bytes / 16;
        d.dst_stride = g.n * d.units;
        d.dst_offset = g.i * d.units;
        d.chunk_start = chunks;
        d.chunks_per_image = ceil_div(d.units, kChunk);
        chunks += g.B * d.chunks_per_image;
    }
    if (a.count == 0) return hipSuccess;
    a.total_chunks = chunks;
    const int cus = device_cus();
    const int64_t resident = int64_t(cus > 0 ? cus : 256);
    const int64_t blocks = chunks < resident ? chunks : resident;
    hipLaunchKernelGGL(refresh_maps_kernel, dim3(unsigned(blocks)), dim3(kMapThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace dp
