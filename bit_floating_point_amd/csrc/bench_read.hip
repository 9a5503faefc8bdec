// Measurement helper for bench.py, not part of libfp4: the attainable rate of a plain
// streaming read of a buffer, the ceiling against which the decode GEMV's HBM rate is
// compared.  Each workgroup of 512 threads reads 32 KiB as four 16-byte nontemporal
// loads per lane, every load instruction 1 KiB contiguous (whole 128-byte lines); the
// loaded words are combined and stored only if they equal a value no input holds, so
// nothing but a few bytes is written.  Offsets past the buffer read zeros (buffer range).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512, kLoads = 4;

__global__ void __launch_bounds__(kThreads) stream_read_kernel(const void* p, int64_t bytes, uint32_t* sink) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
    const uint32_t base = (uint32_t)blockIdx.x * (kThreads * kLoads * 16) + threadIdx.x * 16;
    uint32_t x = 0;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; i++)
        v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + i * kThreads * 16, 0, 2));
#pragma unroll
    for (int i = 0; i < kLoads; i++) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

// Read `bytes` (< 2^31) bytes at p on `stream`; sink: device uint32 scratch.  Returns the
// hipError_t of the launch.
extern "C" int fp4bench_stream_read(const void* p, int64_t bytes, uint32_t* sink, void* stream) {
    if (bytes <= 0 || bytes >= 0x7fff0000) return (int)hipErrorInvalidValue;
    const int64_t per = (int64_t)kThreads * kLoads * 16;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)((bytes + per - 1) / per)), dim3(kThreads), 0,
                       (hipStream_t)stream, p, bytes, sink);
    return (int)hipGetLastError();
}
