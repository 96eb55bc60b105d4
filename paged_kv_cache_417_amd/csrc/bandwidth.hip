// bandwidth.hip — a plain read stream, the measured ceiling beside which the
// decode kernels' HBM rates are reported.  Not part of attention.
//
// Every byte of the buffer is read once with 16-byte non-temporal loads
// (four in flight per thread, grid-stride), and the 32-bit words are folded
// with XOR into one word per workgroup, so the loads cannot be elided and
// the result is checkable: the XOR of all the sink words is the XOR of all
// the buffer's words, whatever the order.
#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4 *__restrict__ src, size_t n,
                                                          uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t s = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        const u32x4 x = (a ^ b) ^ (c ^ d);
        s ^= (x[0] ^ x[1]) ^ (x[2] ^ x[3]);
    }
    for (; i < n; i += stride) {
        const u32x4 x = src[i];
        s ^= (x[0] ^ x[1]) ^ (x[2] ^ x[3]);
    }
    // wave fold, then one word per wave into LDS, one per workgroup out
    for (int o = 32; o > 0; o >>= 1) s ^= (uint32_t)__shfl_xor((int)s, o, 64);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (part[0] ^ part[1]) ^ (part[2] ^ part[3]);
}

}  // namespace

int launch_read_stream(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    hipLaunchKernelGGL(read_stream_kernel, dim3(kReadStreamBlocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const u32x4 *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}

}  // namespace pa
