// Streaming reference for the benchmark (not part of the decode library): a
// kernel that only reads, with the decode launch's grid shape.  Each of the
// `blocks` blocks of `threads` threads reads its own contiguous run of
// `block_bytes` bytes (a multiple of threads * 16) with 16-byte non-temporal
// loads, up to 16 in flight per thread (as the decode kernel issues its tile
// and log loads before using any), folds them into one value per
// thread and stores it, so no load can be dropped.  Timed next to a decode
// launch of the same blocks and bytes, it shows how fast this GPU moves that
// many bytes in that grid when nothing else is done.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

template <int NT>
__global__ void __launch_bounds__(NT) stream_read_kernel(const char *src, float *dst, uint32_t block_bytes) {
    constexpr int U = 16;                       // 16-byte loads in flight per thread
    const char *b = src + (size_t)blockIdx.x * block_bytes;
    const uint32_t loads = block_bytes / (NT * 16);
    float acc = 0.f;
    for (uint32_t j = 0; j < loads; j += U) {   // a batch of up to U loads, all issued before any is used
        v4u32 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            r[u] = v4u32{0u, 0u, 0u, 0u};
            if (j + u < loads)
                r[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4u32 *>(b + ((size_t)(j + u) * NT + threadIdx.x) * 16));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc += __uint_as_float(r[u].x) + __uint_as_float(r[u].y) + __uint_as_float(r[u].z) + __uint_as_float(r[u].w);
    }
    dst[(size_t)blockIdx.x * NT + threadIdx.x] = acc;
}

}  // namespace

// src: device, blocks * block_bytes bytes; dst: device, blocks * threads floats.
// threads in {64, 128, 256}; block_bytes a positive multiple of threads * 16.
// Returns 0, or -1 for bad arguments, or the HIP error of the launch.
extern "C" int dl_probe_stream_read(const void *src, float *dst, int32_t blocks, int32_t threads,
                                    uint32_t block_bytes, void *stream) {
    if (!src || !dst || blocks < 1 || block_bytes == 0 || block_bytes % (uint32_t)(threads * 16)) return -1;
    const hipStream_t s = (hipStream_t)stream;
    const char *p = static_cast<const char *>(src);
    switch (threads) {
    case 64: stream_read_kernel<64><<<blocks, 64, 0, s>>>(p, dst, block_bytes); break;
    case 128: stream_read_kernel<128><<<blocks, 128, 0, s>>>(p, dst, block_bytes); break;
    case 256: stream_read_kernel<256><<<blocks, 256, 0, s>>>(p, dst, block_bytes); break;
    default: return -1;
    }
    return (int)hipGetLastError();
}
