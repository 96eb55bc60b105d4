// cache_ops.hip — cache write (scatter new K/V rows into their slots) and
// whole-block copy for copy-on-write.
//
// Sources (page title, section):
//   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1 — a new token only needs
//        its block and the block table updated.
//   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §2.1 — K and V
//        are two contiguous regions per block; copy-on-write shares prefixes.
//
// Layout: k_cache [NB][Hkv][BS][D] (token rows contiguous),
//         v_cache [NB][Hkv][D][BS] (dimension rows contiguous).
// Both kernels only move bits: no value is converted.
#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

// One thread per (token, kv head, 16-byte chunk of the head's row).  The K
// chunk is a single 16-byte store; the V chunk's elements go to VEC different
// dimension rows at the token's column.
template <typename T>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const T *__restrict__ k_new, const T *__restrict__ v_new, T *__restrict__ k_cache,
    T *__restrict__ v_cache, const int64_t *__restrict__ slots, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks) {
    constexpr int VEC = 16 / sizeof(T);
    const int32_t chunks = head_dim / VEC;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
    if (idx >= total) return;
    const int32_t c = (int32_t)(idx % chunks);
    const int64_t th = idx / chunks;  // token * Hkv + head
    const int32_t h = (int32_t)(th % num_kv_heads);
    const int64_t t = th / num_kv_heads;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
    const int64_t b = slot / block_size;
    const int32_t o = (int32_t)(slot % block_size);
    const int64_t src = th * head_dim + (int64_t)c * VEC;
    const int64_t bh = b * num_kv_heads + h;

    st16(k_cache + (bh * block_size + o) * head_dim + (int64_t)c * VEC, ld16(k_new + src));

    union {
        u32x4 v;
        T e[VEC];
    } u;
    u.v = ld16(v_new + src);
    T *vcol = v_cache + (bh * head_dim + (int64_t)c * VEC) * block_size + o;
#pragma unroll
    for (int e = 0; e < VEC; ++e) vcol[(int64_t)e * block_size] = u.e[e];
}

// One thread per 16 bytes of one pair's K or V block region (both regions are
// Hkv*BS*D contiguous elements).
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    char *__restrict__ k_cache, char *__restrict__ v_cache, const int32_t *__restrict__ src_dst,
    int32_t num_pairs, int64_t block_bytes, int32_t num_blocks) {
    const int64_t per_region = block_bytes / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)num_pairs * 2 * per_region) return;
    const int64_t chunk = idx % per_region;
    const int64_t pr = idx / per_region;
    const int32_t pair = (int32_t)(pr >> 1);
    char *base = (pr & 1) ? v_cache : k_cache;
    const int32_t src = src_dst[2 * pair];
    const int32_t dst = src_dst[2 * pair + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    st16(base + dst * block_bytes + chunk * 16, ld16(base + src * block_bytes + chunk * 16));
}

}  // namespace

int launch_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                       void *stream) {
    if (num_tokens == 0) return 0;
    const int vec = dtype == PA_DTYPE_BF16 ? 8 : 4;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_dim / vec);
    const dim3 grid((unsigned)((total + 255) / 256));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dtype == PA_DTYPE_BF16) {
        hipLaunchKernelGGL(cache_write_kernel<uint16_t>, grid, dim3(256), 0, s,
                           (const uint16_t *)k_new, (const uint16_t *)v_new, (uint16_t *)k_cache,
                           (uint16_t *)v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                           block_size, num_blocks);
    } else {
        hipLaunchKernelGGL(cache_write_kernel<uint32_t>, grid, dim3(256), 0, s,
                           (const uint32_t *)k_new, (const uint32_t *)v_new, (uint32_t *)k_cache,
                           (uint32_t *)v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                           block_size, num_blocks);
    }
    return (int)hipGetLastError();
}

int launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_dst, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, pa_dtype dtype, void *stream) {
    if (num_pairs == 0) return 0;
    const int64_t elem = dtype == PA_DTYPE_BF16 ? 2 : 4;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem;
    const int64_t total = (int64_t)num_pairs * 2 * (block_bytes / 16);
    const dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (char *)k_cache, (char *)v_cache, src_dst, num_pairs, block_bytes,
                       num_blocks);
    return (int)hipGetLastError();
}

}  // namespace pa
