// noalloc.hip — pa_decode without a caller workspace, for callers that
// cannot allocate device memory (code under graph capture, serving loops
// that forbid allocation).
//
// The split-K partials live in `scratch`, a file-scope device array that
// each GPU the library runs on holds from module load until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array: its device address comes from hipGetSymbolAddress, taken once per
// device (with that device current) and kept in `g_scratch`.  Only that
// address ever reaches a kernel.  No call here allocates or frees device
// memory.  Nothing in the workspace must start at zero: the reduce reads
// only partials that the same call's partition kernel wrote.
#include <mutex>

#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // PA_DECODE_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == PA_DECODE_NOALLOC_SCRATCH_BYTES, "header and library disagree");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];  // per device: the address of its copy of `scratch`

// Device address of the current device's `scratch`, looked up on the first
// call on that device; nullptr (with the error recorded) on failure.
void *device_scratch(const char *fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        pa::fail(PA_ERR_DEVICE, "%s: no current device (hip error %d, device %d)", fn, (int)e,
                 dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            pa::fail(PA_ERR_DEVICE, "%s: scratch address on device %d (hip error %d)", fn, dev,
                     (int)e);
            return nullptr;
        }
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(float *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, int32_t block_table_stride,
                            const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale, int32_t max_context_len,
                            int32_t partition_size, pa_dtype dtype, uint32_t flags,
                            void *stream) {
    const char *fn = "pa_decode_noalloc";
    const size_t need = pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 block_size, max_context_len, partition_size);
    // (size_t)-1 (invalid sizes) goes on to pa_decode_ex, which names the
    // bad argument
    if (need != (size_t)-1 && need > kScratchBytes)
        return pa::fail(PA_ERR_UNSUPPORTED,
                        "%s: the split-K partials need %zu bytes, the built-in scratch holds %zu "
                        "(fewer sequences, a shorter max_context_len or a larger partition_size "
                        "fit; pa_decode_ex takes a workspace of any size)",
                        fn, need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0 && need != (size_t)-1) {
        ws = device_scratch(fn);
        if (!ws) return PA_ERR_DEVICE;
    }
    return pa_decode_ex(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        scale, max_context_len, partition_size, ws, ws ? kScratchBytes : 0, dtype,
                        flags, stream);
}

}  // extern "C"
