/*
 * oracle.h — fp64 CPU oracle for paged-KV attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this code; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no header, helper or constant with
 * the HIP path.
 *
 * Sources (page title, section):
 *   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》
 *   [VF] 《大模型推理：vLLM大模型推理框架（附下载）》
 *   [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》
 *   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》
 *
 * Every function computes the plain definition, element by element, in double
 * precision.  Storage layout is passed as element strides, so the oracle does
 * not depend on how the product lays K and V out inside a block.
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };  /* FP8: OCP E4M3 codes */

/* Element strides of one paged pool: element (block b, kv head h, row r, dim d)
 * sits at b*block + h*head + r*row + d*dim. */
typedef struct {
    int64_t block, head, row, dim;
} orc_strides;

/* OCP E4M3 code -> value (NaN for S.1111.111), and value -> nearest code
 * (ties to the even code, saturating at +-448, NaN -> 0x7F). */
double orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(float x);

/* Quantizing cache write: code = nearest E4M3 of (x / scale) in binary32. */
void orc_cache_write_fp8(const void *k_new, const void *v_new, int in_dtype,
                         uint8_t *k_cache, orc_strides ks, uint8_t *v_cache, orc_strides vs,
                         const int64_t *slot_mapping, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         float k_scale, float v_scale);

/* Widen one stored element (fp32, bf16 bits or an E4M3 code) to double, exactly. */
double orc_widen(const void *base, int64_t index, int dtype);

/* Un-page one sequence of one kv head: out[t][d] for t < len. */
void orc_unpage(const void *cache, orc_strides st, int dtype,
                const int32_t *table, int32_t block_size, int32_t len,
                int32_t head, int32_t head_dim, double *out);

/* softmax(scale * q K^T) V for one query row over L contiguous keys. */
void orc_attention(const double *q, const double *K, const double *V,
                   int32_t L, int32_t head_dim, double scale, double *out);

/* Paged decode: out[s][h][:] for every sequence s and query head h. */
void orc_decode(double *out, const void *q, int q_dtype,
                const void *k_cache, orc_strides ks,
                const void *v_cache, orc_strides vs, int kv_dtype,
                const int32_t *block_tables, int32_t table_stride,
                const int32_t *context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, double scale, double k_scale, double v_scale);

/* Paged causal prefill over a chunk of new query rows per request. */
void orc_prefill(double *out, const void *q, int q_dtype,
                 const void *k_cache, orc_strides ks,
                 const void *v_cache, orc_strides vs, int kv_dtype,
                 const int32_t *block_tables, int32_t table_stride,
                 const int32_t *cu_q_lens, const int32_t *context_lens,
                 int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t block_size, double scale, double k_scale,
                 double v_scale);

/* Scatter new K/V rows [T][Hkv][D] into their slots, byte for byte. */
void orc_cache_write(const void *k_new, const void *v_new,
                     void *k_cache, orc_strides ks,
                     void *v_cache, orc_strides vs,
                     const int64_t *slot_mapping, int32_t num_tokens,
                     int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t elem_size);

/* Copy every element of block src to block dst, for K and V, all heads. */
void orc_copy_blocks(void *k_cache, orc_strides ks, void *v_cache, orc_strides vs,
                     const int32_t *src_dst, int32_t num_pairs,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t elem_size);

/* Copy block src of (src_k, src_v) to block dst of (dst_k, dst_v), all heads. */
void orc_swap_blocks(const void *src_k, orc_strides sks, const void *src_v, orc_strides svs,
                     void *dst_k, orc_strides dks, void *dst_v, orc_strides dvs,
                     const int32_t *src_dst, int32_t num_pairs,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t elem_size);

#ifdef __cplusplus
}
#endif
#endif
