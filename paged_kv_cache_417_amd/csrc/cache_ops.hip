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
// The bf16/fp32 write and the block copies only move bits; the fp8 write
// quantizes to OCP E4M3 codes with one scale per cache.
#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int32_t kRunBatch = 256;  // tokens per call from which V is written by runs

// Index arithmetic of the one-thread-per-16-byte-chunk paths: the grid is
// bounded by 2^32 threads, so indices are 32-bit, and head_dim / VEC and the
// block size are powers of two (shifts, not divisions).
struct ChunkIndex {
    uint32_t th;  // token * Hkv + head
    int32_t h, c;
};
template <typename T>
__device__ __forceinline__ ChunkIndex chunk_index(uint32_t idx, int32_t num_kv_heads,
                                                  int32_t head_dim) {
    constexpr int VEC = 16 / sizeof(T);
    const uint32_t cshift = __builtin_ctz((uint32_t)(head_dim / VEC));
    const uint32_t th = idx >> cshift;
    return ChunkIndex{th, (int32_t)(th % (uint32_t)num_kv_heads),
                      (int32_t)(idx & ((1u << cshift) - 1))};
}

// K: one thread per (token, kv head, 16-byte chunk of the head's row): one
// 16-byte store into the token's row of its block.  The row is loaded before
// the slot is known, so the two loads overlap.
template <typename T>
__device__ __forceinline__ void write_k(const T *__restrict__ k_new, T *__restrict__ k_cache,
                                        const int64_t *__restrict__ slots, int64_t idx,
                                        int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks) {
    constexpr int VEC = 16 / sizeof(T);
    if (idx >= (int64_t)num_tokens * num_kv_heads * (head_dim / VEC)) return;
    const ChunkIndex ci = chunk_index<T>((uint32_t)idx, num_kv_heads, head_dim);
    const u32x4 row = ld16(k_new + (int64_t)ci.th * head_dim + ci.c * VEC);
    const int64_t slot = slots[ci.th / (uint32_t)num_kv_heads];
    if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
    const uint32_t bshift = __builtin_ctz((uint32_t)block_size);
    const int64_t b = slot >> bshift;
    const int32_t o = (int32_t)(slot & (block_size - 1));
    st16(k_cache + ((b * num_kv_heads + ci.h) * block_size + o) * head_dim + ci.c * VEC, row);
}

// V (dimension rows of a block): one thread per (run of VEC consecutive
// tokens, kv head, dim).  Lanes walk the dims, so the reads of each token's
// row are coalesced.  When the run's slots are consecutive and start at a
// multiple of VEC -- the usual case for a prompt chunk, whose tokens fill
// blocks in order -- the run lands as one 16-byte store into the dim row;
// otherwise (decode steps: one token per sequence) each token's element is
// stored on its own.
template <typename T>
__device__ __forceinline__ void write_v(const T *__restrict__ v_new, T *__restrict__ v_cache,
                                        const int64_t *__restrict__ slots, int64_t idx,
                                        int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks) {
    constexpr int VEC = 16 / sizeof(T);
    const int64_t runs = ((int64_t)num_tokens + VEC - 1) / VEC;
    if (idx >= runs * num_kv_heads * head_dim) return;
    const int32_t d = (int32_t)(idx % head_dim);
    const int64_t rh = idx / head_dim;
    const int32_t h = (int32_t)(rh % num_kv_heads);
    const int64_t t0 = (rh / num_kv_heads) * VEC;
    const int64_t limit = (int64_t)num_blocks * block_size;
    const int32_t n = (int32_t)min((int64_t)VEC, (int64_t)num_tokens - t0);
    const int64_t s0 = slots[t0];
    bool packed = n == VEC && s0 >= 0 && s0 + VEC <= limit && s0 % VEC == 0;
    union {
        u32x4 v;
        T e[VEC];
    } u;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        if (i < n) {
            u.e[i] = v_new[((t0 + i) * num_kv_heads + h) * head_dim + d];
            if (i > 0) packed = packed && slots[t0 + i] == s0 + i;
        }
    }
    if (packed) {
        const int64_t b = s0 / block_size;
        const int32_t o = (int32_t)(s0 % block_size);
        st16(v_cache + ((b * num_kv_heads + h) * head_dim + d) * block_size + o, u.v);
        return;
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        if (i >= n) break;
        const int64_t slot = slots[t0 + i];
        if (slot < 0 || slot >= limit) continue;
        const int64_t b = slot / block_size;
        const int32_t o = (int32_t)(slot % block_size);
        v_cache[((b * num_kv_heads + h) * head_dim + d) * block_size + o] = u.e[i];
    }
}

// V, one thread per (token, kv head, 16-byte chunk): one 16-byte load of
// the token's row and VEC element stores into VEC dim rows.  Cheapest when
// no two tokens of the batch share a block row (decode steps).
template <typename T>
__device__ __forceinline__ void write_v_tokens(const T *__restrict__ v_new,
                                               T *__restrict__ v_cache,
                                               const int64_t *__restrict__ slots, int64_t idx,
                                               int32_t num_tokens, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size,
                                               int32_t num_blocks) {
    constexpr int VEC = 16 / sizeof(T);
    if (idx >= (int64_t)num_tokens * num_kv_heads * (head_dim / VEC)) return;
    const ChunkIndex ci = chunk_index<T>((uint32_t)idx, num_kv_heads, head_dim);
    union {
        u32x4 v;
        T e[VEC];
    } u;
    u.v = ld16(v_new + (int64_t)ci.th * head_dim + ci.c * VEC);  // overlaps the slot load
    const int64_t slot = slots[ci.th / (uint32_t)num_kv_heads];
    if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
    const uint32_t bshift = __builtin_ctz((uint32_t)block_size);
    const int64_t b = slot >> bshift;
    const int32_t o = (int32_t)(slot & (block_size - 1));
    T *col = v_cache + ((b * num_kv_heads + ci.h) * head_dim + ci.c * VEC) * block_size + o;
#pragma unroll
    for (int e = 0; e < VEC; ++e) col[(int64_t)e * block_size] = u.e[e];
}

// Workgroups [0, k_groups) write K, the rest write V, by runs or by tokens.
template <typename T, bool RUNS>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const T *__restrict__ k_new, const T *__restrict__ v_new, T *__restrict__ k_cache,
    T *__restrict__ v_cache, const int64_t *__restrict__ slots, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    uint32_t k_groups) {
    if (blockIdx.x < k_groups) {
        write_k<T>(k_new, k_cache, slots, (int64_t)blockIdx.x * 256 + threadIdx.x, num_tokens,
                   num_kv_heads, head_dim, block_size, num_blocks);
    } else if (RUNS) {
        write_v<T>(v_new, v_cache, slots, (int64_t)(blockIdx.x - k_groups) * 256 + threadIdx.x,
                   num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
    } else {
        write_v_tokens<T>(v_new, v_cache, slots,
                          (int64_t)(blockIdx.x - k_groups) * 256 + threadIdx.x, num_tokens,
                          num_kv_heads, head_dim, block_size, num_blocks);
    }
}

// Nearest E4M3 codes of x / scale for four values, packed lowest first.  The
// division is binary32, correctly rounded; the hardware conversion rounds to
// nearest even but turns magnitudes past 448 into NaN, so values are clamped
// to +-448 first (saturation), and a NaN input gets the code 0x7F.
__device__ __forceinline__ uint32_t e4m3_quant4(const float *x, float scale) {
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(x[i] / scale, -448.f), 448.f);
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)w, true);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (x[i] != x[i]) w = (w & ~(0xffu << (8 * i))) | (0x7fu << (8 * i));
    return w;
}

// fp8 cache write: one thread per (token, kv head, 16 dims).  K: the 16
// codes are one 16-byte store into the token's row; V: one byte into each of
// the 16 dim rows.
template <typename T>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const T *__restrict__ k_new, const T *__restrict__ v_new, uint8_t *__restrict__ k_cache,
    uint8_t *__restrict__ v_cache, const int64_t *__restrict__ slots, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    float k_scale, float v_scale) {
    const int32_t chunks = head_dim / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)num_tokens * num_kv_heads * chunks) return;
    const int32_t c = (int32_t)(idx % chunks);
    const int64_t th = idx / chunks;  // token * Hkv + head
    const int32_t h = (int32_t)(th % num_kv_heads);
    const int64_t slot = slots[th / num_kv_heads];
    if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
    const int64_t b = slot / block_size;
    const int32_t o = (int32_t)(slot % block_size);
    const int64_t src = th * head_dim + (int64_t)c * 16;
    float kx[16], vx[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        kx[i] = (float)k_new[src + i];
        vx[i] = (float)v_new[src + i];
    }
    u32x4 kw;
#pragma unroll
    for (int i = 0; i < 4; ++i) kw[i] = e4m3_quant4(kx + 4 * i, k_scale);
    st16(k_cache + ((b * num_kv_heads + h) * block_size + o) * head_dim + (int64_t)c * 16, kw);
    uint8_t *vrow = v_cache + ((b * num_kv_heads + h) * head_dim + (int64_t)c * 16) * block_size + o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t vw = e4m3_quant4(vx + 4 * i, v_scale);
#pragma unroll
        for (int e = 0; e < 4; ++e) vrow[(int64_t)(4 * i + e) * block_size] = (uint8_t)(vw >> (8 * e));
    }
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

// Block copy between two pools (swap out: device -> pinned host; swap in:
// host -> device).  One thread per 16 bytes of a block region, so the PCIe
// side sees long runs of 16-byte accesses.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const char *__restrict__ src_k, const char *__restrict__ src_v, char *__restrict__ dst_k,
    char *__restrict__ dst_v, const int32_t *__restrict__ src_dst, int32_t num_pairs,
    int64_t block_bytes, int32_t src_blocks, int32_t dst_blocks) {
    const int64_t per_region = block_bytes / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)num_pairs * 2 * per_region) return;
    const int64_t chunk = idx % per_region;
    const int64_t pr = idx / per_region;
    const int32_t pair = (int32_t)(pr >> 1);
    const int32_t src = src_dst[2 * pair];
    const int32_t dst = src_dst[2 * pair + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
    const char *from = (pr & 1) ? src_v : src_k;
    char *to = (pr & 1) ? dst_v : dst_k;
    st16(to + dst * block_bytes + chunk * 16, ld16(from + src * block_bytes + chunk * 16));
}

}  // namespace

int launch_cache_write(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                       void *stream) {
    if (num_tokens == 0) return 0;
    const int vec = dtype == PA_DTYPE_BF16 ? 8 : 4;
    // Batches of many tokens are mostly prompt chunks whose slots run in
    // order; small ones are decode steps (one token per sequence).  Both V
    // paths are exact for any slots: the choice only affects speed.
    const bool runs = num_tokens >= kRunBatch;
    const int64_t k_threads = (int64_t)num_tokens * num_kv_heads * (head_dim / vec);
    const int64_t v_threads = runs ? ((int64_t)num_tokens + vec - 1) / vec * num_kv_heads * head_dim
                                   : k_threads;
    const int64_t k_groups = (k_threads + 255) / 256;
    const int64_t groups = k_groups + (v_threads + 255) / 256;
    if (!grid_fits(groups * 256)) return kLaunchTooLarge;
    const dim3 grid((unsigned)groups);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#define PA_LAUNCH(T, R)                                                                         \
    hipLaunchKernelGGL((cache_write_kernel<T, R>), grid, dim3(256), 0, s, (const T *)k_new,     \
                       (const T *)v_new, (T *)k_cache, (T *)v_cache, slot_mapping, num_tokens, \
                       num_kv_heads, head_dim, block_size, num_blocks, (uint32_t)k_groups)
    if (dtype == PA_DTYPE_BF16) {
        if (runs) PA_LAUNCH(uint16_t, true); else PA_LAUNCH(uint16_t, false);
    } else {
        if (runs) PA_LAUNCH(uint32_t, true); else PA_LAUNCH(uint32_t, false);
    }
#undef PA_LAUNCH
    return (int)hipGetLastError();
}

int launch_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_dst, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, pa_dtype dtype, void *stream) {
    if (num_pairs == 0) return 0;
    const int64_t elem = dtype == PA_DTYPE_BF16 ? 2 : dtype == PA_DTYPE_FP8_E4M3 ? 1 : 4;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem;
    const int64_t total = (int64_t)num_pairs * 2 * (block_bytes / 16);
    if (!grid_fits(total)) return kLaunchTooLarge;
    const dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (char *)k_cache, (char *)v_cache, src_dst, num_pairs, block_bytes,
                       num_blocks);
    return (int)hipGetLastError();
}

int launch_swap_blocks(const void *src_k, const void *src_v, int32_t src_blocks, void *dst_k,
                       void *dst_v, int32_t dst_blocks, const int32_t *src_dst,
                       int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, pa_dtype dtype, void *stream) {
    if (num_pairs == 0) return 0;
    const int64_t elem = dtype == PA_DTYPE_BF16 ? 2 : dtype == PA_DTYPE_FP8_E4M3 ? 1 : 4;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem;
    const int64_t total = (int64_t)num_pairs * 2 * (block_bytes / 16);
    if (!grid_fits(total)) return kLaunchTooLarge;
    const dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (const char *)src_k, (const char *)src_v, (char *)dst_k, (char *)dst_v,
                       src_dst, num_pairs, block_bytes, src_blocks, dst_blocks);
    return (int)hipGetLastError();
}

int launch_cache_write_fp8(const void *k_new, const void *v_new, pa_dtype in_dtype,
                           void *k_cache, void *v_cache, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, float k_scale,
                           float v_scale, void *stream) {
    if (num_tokens == 0) return 0;
    const int64_t threads = (int64_t)num_tokens * num_kv_heads * (head_dim / 16);
    const int64_t groups = (threads + 255) / 256;
    if (!grid_fits(threads)) return kLaunchTooLarge;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (in_dtype == PA_DTYPE_BF16)
        hipLaunchKernelGGL(cache_write_fp8_kernel<__bf16>, dim3((unsigned)groups), dim3(256), 0, s,
                           (const __bf16 *)k_new, (const __bf16 *)v_new, (uint8_t *)k_cache,
                           (uint8_t *)v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                           block_size, num_blocks, k_scale, v_scale);
    else
        hipLaunchKernelGGL(cache_write_fp8_kernel<float>, dim3((unsigned)groups), dim3(256), 0, s,
                           (const float *)k_new, (const float *)v_new, (uint8_t *)k_cache,
                           (uint8_t *)v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                           block_size, num_blocks, k_scale, v_scale);
    return (int)hipGetLastError();
}

}  // namespace pa
