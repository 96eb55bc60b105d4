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

/* OCP 8-bit floating point, E4M3 variant: a sign bit, 4 exponent bits with
 * bias 7 and 3 mantissa bits.  Exponent field 0 holds the subnormals
 * m * 2^-9; otherwise the value is (1 + m/8) * 2^(e-7).  There are no
 * infinities: S.1111.111 is NaN, so the largest magnitude is 448. */
double orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* The E4M3 code nearest to x, by search over every finite code; a tie goes
 * to the code whose last bit is 0 (round half to even).  Magnitudes beyond
 * 448, infinities included, saturate to +-448; NaN gives 0x7F. */
uint8_t orc_e4m3_encode(float x)
{
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isinf(x)) return (uint8_t)(sign | 0x7E);
    double a = fabs((double)x);
    int best = 0;
    double best_err = a;  /* code 0 is +0 */
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs(orc_e4m3_decode((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

double orc_widen(const void *base, int64_t index, int dtype)
{
    if (dtype == ORC_FP8) {
        uint8_t c;
        memcpy(&c, (const char *)base + index, 1);
        return orc_e4m3_decode(c);
    }
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
                int32_t block_size, double scale, double k_scale, double v_scale)
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
            /* stored values times the cache's scale (exact in double) */
            for (int64_t i = 0; i < (int64_t)L * head_dim; ++i) {
                K[i] *= k_scale;
                V[i] *= v_scale;
            }
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
                 int32_t head_dim, int32_t block_size, double scale, double k_scale,
                 double v_scale)
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
            for (int64_t e = 0; e < (int64_t)ctx * head_dim; ++e) {  /* cache scales */
                K[e] *= k_scale;
                V[e] *= v_scale;
            }
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

/* fp8 cache write: each element of the new rows is divided by its cache's
 * scale in binary32 (correctly rounded) and stored as the nearest E4M3 code
 * (orc_e4m3_encode).  Slots and layout as in orc_cache_write. */
void orc_cache_write_fp8(const void *k_new, const void *v_new, int in_dtype,
                         uint8_t *k_cache, orc_strides ks, uint8_t *v_cache, orc_strides vs,
                         const int64_t *slot_mapping, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         float k_scale, float v_scale)
{
    for (int32_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t b = slot / block_size, r = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; ++h)
            for (int32_t d = 0; d < head_dim; ++d) {
                int64_t src = ((int64_t)t * num_kv_heads + h) * head_dim + d;
                float kx = (float)orc_widen(k_new, src, in_dtype);
                float vx = (float)orc_widen(v_new, src, in_dtype);
                k_cache[b * ks.block + h * ks.head + r * ks.row + d * ks.dim] =
                    orc_e4m3_encode(kx / k_scale);
                v_cache[b * vs.block + h * vs.head + r * vs.row + d * vs.dim] =
                    orc_e4m3_encode(vx / v_scale);
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
