/*
 * oracle.c — fp64 CPU oracle for paged-KV attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the benchmark's
 * CPU-baseline leg; never by the product path.  Plain loops, no blocking, no
 * fusion, no reordering beyond the definitions below.
 *
 * Sources (page title, section):
 *   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》
 *   [VF] 《大模型推理：vLLM大模型推理框架（附下载）》
 *   [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》
 *   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

double orc_widen(const void *base, int64_t index, int dtype)
{
    if (dtype == ORC_F32) {
        float f;
        memcpy(&f, (const char *)base + index * 4, 4);
        return (double)f;
    }
    /* bf16 is the top half of an IEEE binary32: shifting the 16 stored bits
       up gives the same value exactly. */
    uint16_t h;
    memcpy(&h, (const char *)base + index * 2, 2);
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Logical position t of a sequence lives in logical block t / block_size at
 * offset t % block_size, and the block table names the physical block
 * ([VF] §1.1 PagedAttention pseudo-code; [VE] §3.1, the block table). */
void orc_unpage(const void *cache, orc_strides st, int dtype,
                const int32_t *table, int32_t block_size, int32_t len,
                int32_t head, int32_t head_dim, double *out)
{
    for (int32_t t = 0; t < len; ++t) {
        int64_t logical_block = t / block_size;
        int64_t offset = t % block_size;
        int64_t physical = table[logical_block];
        for (int32_t d = 0; d < head_dim; ++d) {
            int64_t idx = physical * st.block + (int64_t)head * st.head +
                          offset * st.row + (int64_t)d * st.dim;
            out[(int64_t)t * head_dim + d] = orc_widen(cache, idx, dtype);
        }
    }
}

/* Attention for one query row: scaling, softmax, weighted sum ([VE] §3.3,
 * the fused attention steps).  Max-subtracted softmax over L keys; L == 0
 * yields zeros (an empty row reads nothing). */
void orc_attention(const double *q, const double *K, const double *V,
                   int32_t L, int32_t head_dim, double scale, double *out)
{
    for (int32_t d = 0; d < head_dim; ++d) out[d] = 0.0;
    if (L <= 0) return;

    double *z = (double *)malloc(sizeof(double) * (size_t)L);
    double m = -INFINITY;
    for (int32_t t = 0; t < L; ++t) {
        double dot = 0.0;
        for (int32_t d = 0; d < head_dim; ++d)
            dot += q[d] * K[(int64_t)t * head_dim + d];
        z[t] = scale * dot;
        if (z[t] > m) m = z[t];
    }
    double l = 0.0;
    for (int32_t t = 0; t < L; ++t) {
        z[t] = exp(z[t] - m);
        l += z[t];
    }
    for (int32_t t = 0; t < L; ++t) {
        double p = z[t] / l;
        for (int32_t d = 0; d < head_dim; ++d)
            out[d] += p * V[(int64_t)t * head_dim + d];
    }
    free(z);
}

/* Decode: one new query row per sequence attends to all context_lens[s]
 * cached keys of that sequence, read through its block table ([VE] §3.1).
 * Query head h reads kv head h / (Hq / Hkv) (contiguous grouping). */
void orc_decode(double *out, const void *q, int q_dtype,
                const void *k_cache, orc_strides ks,
                const void *v_cache, orc_strides vs, int kv_dtype,
                const int32_t *block_tables, int32_t table_stride,
                const int32_t *context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, double scale)
{
    int32_t group = num_q_heads / num_kv_heads;
    int32_t max_len = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (context_lens[s] > max_len) max_len = context_lens[s];
    size_t rows = max_len > 0 ? (size_t)max_len : 1;
    double *K = (double *)malloc(sizeof(double) * rows * (size_t)head_dim);
    double *V = (double *)malloc(sizeof(double) * rows * (size_t)head_dim);
    double *qv = (double *)malloc(sizeof(double) * (size_t)head_dim);

    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t *table = block_tables + (int64_t)s * table_stride;
        int32_t L = context_lens[s];
        for (int32_t h = 0; h < num_q_heads; ++h) {
            int32_t kvh = h / group;
            orc_unpage(k_cache, ks, kv_dtype, table, block_size, L, kvh, head_dim, K);
            orc_unpage(v_cache, vs, kv_dtype, table, block_size, L, kvh, head_dim, V);
            int64_t qoff = ((int64_t)s * num_q_heads + h) * head_dim;
            for (int32_t d = 0; d < head_dim; ++d)
                qv[d] = orc_widen(q, qoff + d, q_dtype);
            orc_attention(qv, K, V, L, head_dim, scale,
                          out + ((int64_t)s * num_q_heads + h) * head_dim);
        }
    }
    free(K);
    free(V);
    free(qv);
}

/* Prefill chunk: request r contributes the new query rows
 * cu_q_lens[r] .. cu_q_lens[r+1]-1.  Its context holds context_lens[r] keys,
 * the chunk's own keys last, so row i sits at absolute position
 * p = context_lens[r] - qlen + i and attends to keys 0..p (causal).  One
 * iteration may mix such chunks with decode rows ([VI] §1, continuous
 * batching). */
void orc_prefill(double *out, const void *q, int q_dtype,
                 const void *k_cache, orc_strides ks,
                 const void *v_cache, orc_strides vs, int kv_dtype,
                 const int32_t *block_tables, int32_t table_stride,
                 const int32_t *cu_q_lens, const int32_t *context_lens,
                 int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t block_size, double scale)
{
    int32_t group = num_q_heads / num_kv_heads;
    int32_t max_len = 1;
    for (int32_t r = 0; r < num_reqs; ++r)
        if (context_lens[r] > max_len) max_len = context_lens[r];
    double *K = (double *)malloc(sizeof(double) * (size_t)max_len * (size_t)head_dim);
    double *V = (double *)malloc(sizeof(double) * (size_t)max_len * (size_t)head_dim);
    double *qv = (double *)malloc(sizeof(double) * (size_t)head_dim);

    for (int32_t r = 0; r < num_reqs; ++r) {
        const int32_t *table = block_tables + (int64_t)r * table_stride;
        int32_t ctx = context_lens[r];
        int32_t q0 = cu_q_lens[r];
        int32_t qlen = cu_q_lens[r + 1] - q0;
        for (int32_t h = 0; h < num_q_heads; ++h) {
            int32_t kvh = h / group;
            orc_unpage(k_cache, ks, kv_dtype, table, block_size, ctx, kvh, head_dim, K);
            orc_unpage(v_cache, vs, kv_dtype, table, block_size, ctx, kvh, head_dim, V);
            for (int32_t i = 0; i < qlen; ++i) {
                int32_t pos = ctx - qlen + i;
                int64_t row = ((int64_t)(q0 + i) * num_q_heads + h) * head_dim;
                for (int32_t d = 0; d < head_dim; ++d)
                    qv[d] = orc_widen(q, row + d, q_dtype);
                orc_attention(qv, K, V, pos + 1, head_dim, scale, out + row);
            }
        }
    }
    free(K);
    free(V);
    free(qv);
}

/* Cache write: token i's K and V rows go to slot slot_mapping[i], i.e.
 * physical block slot / block_size at offset slot % block_size ([VE] §3.1:
 * a new token only needs its block and the block table updated).  A negative
 * slot means "no write". */
void orc_cache_write(const void *k_new, const void *v_new,
                     void *k_cache, orc_strides ks,
                     void *v_cache, orc_strides vs,
                     const int64_t *slot_mapping, int32_t num_tokens,
                     int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t elem_size)
{
    for (int32_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        int64_t b = slot / block_size;
        int64_t o = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            for (int32_t d = 0; d < head_dim; ++d) {
                int64_t src = ((int64_t)i * num_kv_heads + h) * head_dim + d;
                int64_t kdst = b * ks.block + (int64_t)h * ks.head + o * ks.row + (int64_t)d * ks.dim;
                int64_t vdst = b * vs.block + (int64_t)h * vs.head + o * vs.row + (int64_t)d * vs.dim;
                memcpy((char *)k_cache + kdst * elem_size, (const char *)k_new + src * elem_size, (size_t)elem_size);
                memcpy((char *)v_cache + vdst * elem_size, (const char *)v_new + src * elem_size, (size_t)elem_size);
            }
        }
    }
}

/* Swap space: whole blocks move between the device pool and a host pool
 * ([NV] best practice 5, preemption to CPU memory; [VI] §2.1 cold blocks to
 * CPU memory).  Block src of the source pools is copied, K and V, every
 * head and row, to block dst of the destination pools. */
void orc_swap_blocks(const void *src_k, orc_strides sks, const void *src_v, orc_strides svs,
                     void *dst_k, orc_strides dks, void *dst_v, orc_strides dvs,
                     const int32_t *src_dst, int32_t num_pairs,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t elem_size)
{
    for (int32_t p = 0; p < num_pairs; ++p) {
        int64_t src = src_dst[2 * p];
        int64_t dst = src_dst[2 * p + 1];
        for (int32_t h = 0; h < num_kv_heads; ++h)
            for (int32_t r = 0; r < block_size; ++r)
                for (int32_t d = 0; d < head_dim; ++d) {
                    memcpy((char *)dst_k + (dst * dks.block + h * dks.head + r * dks.row +
                                            d * dks.dim) * elem_size,
                           (const char *)src_k + (src * sks.block + h * sks.head + r * sks.row +
                                                  d * sks.dim) * elem_size,
                           (size_t)elem_size);
                    memcpy((char *)dst_v + (dst * dvs.block + h * dvs.head + r * dvs.row +
                                            d * dvs.dim) * elem_size,
                           (const char *)src_v + (src * svs.block + h * svs.head + r * svs.row +
                                                  d * svs.dim) * elem_size,
                           (size_t)elem_size);
                }
    }
}

/* Copy-on-write: before a sequence writes into a block it shares, the whole
 * block (K and V, every head, every row) is copied to a private block
 * ([VI] §2.1, COW for prefix sharing). */
void orc_copy_blocks(void *k_cache, orc_strides ks, void *v_cache, orc_strides vs,
                     const int32_t *src_dst, int32_t num_pairs,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t elem_size)
{
    for (int32_t p = 0; p < num_pairs; ++p) {
        int64_t src = src_dst[2 * p];
        int64_t dst = src_dst[2 * p + 1];
        for (int32_t h = 0; h < num_kv_heads; ++h)
            for (int32_t r = 0; r < block_size; ++r)
                for (int32_t d = 0; d < head_dim; ++d) {
                    int64_t ko = (int64_t)h * ks.head + (int64_t)r * ks.row + (int64_t)d * ks.dim;
                    int64_t vo = (int64_t)h * vs.head + (int64_t)r * vs.row + (int64_t)d * vs.dim;
                    memcpy((char *)k_cache + (dst * ks.block + ko) * elem_size,
                           (const char *)k_cache + (src * ks.block + ko) * elem_size, (size_t)elem_size);
                    memcpy((char *)v_cache + (dst * vs.block + vo) * elem_size,
                           (const char *)v_cache + (src * vs.block + vo) * elem_size, (size_t)elem_size);
                }
    }
}
