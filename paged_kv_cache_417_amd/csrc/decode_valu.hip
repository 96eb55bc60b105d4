// decode_valu.hip — paged decode attention on the vector ALU, for fp32 KV
// (and bf16 as a second, independent device implementation), any group size
// up to 16.  One wave per (sequence, kv head, partition).
//
// Sources (page title, section):
//   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1 — block-table walk over
//        scattered blocks; §3.3 — scaling, softmax, weighted sum in one kernel.
//   [VF] 《大模型推理：vLLM大模型推理框架（附下载）》 §1.1 — independent
//        segments (split-K partitions).
//
// Per 16-token step (a step never straddles a block: BS is a multiple of 16):
//   q.k : lane = 4*r + c handles token r of the step and the c-th quarter of
//         the head dims with 16-byte loads; the four partial dots of a token
//         are summed with two DPP quad exchanges.  Scores go to LDS.
//   online softmax : every lane reads the step's scores of each head from LDS
//         (broadcast reads), so the running max and sum are wave-uniform.
//   P V : lane owns dims d = lane (+64); V's dimension-major rows give it the
//         step's 16 tokens of its dims contiguously.
// Tokens at or past the context length get a -inf score and are skipped in
// P V, so poisoned rows never reach the output.
#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

template <typename T>
__device__ __forceinline__ void widen16(const T *p, float *out);

template <>
__device__ __forceinline__ void widen16<uint32_t>(const uint32_t *p, float *out) {
    const u32x4 v = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}

template <>
__device__ __forceinline__ void widen16<uint16_t>(const uint16_t *p, float *out) {
    const u32x4 v = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = bf16_lo(v[i]);
        out[2 * i + 1] = bf16_hi(v[i]);
    }
}

constexpr int kMaxGroup = 16;

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
    constexpr int QD = D / 4;            // dims per lane in q.k
    constexpr int DPL = D / 64;          // dims per lane in P V
    const int BS = p.block_size;
    const DecodeItem item = decode_item(blockIdx.x, p.num_kv_heads, p.num_seqs);
    const int kvh = item.kvh;
    const int s = item.seq;
    const int lane = threadIdx.x;
    const int r = lane >> 2, c = lane & 3;

    const int32_t L = p.context_lens[s];
    const int32_t nb = (L + BS - 1) / BS;
    const bool bad_len = L < 0 || L > p.max_context_len || nb > p.table_stride;
    const int32_t np = bad_len ? 1 : max(1, (L + p.partition_size - 1) / p.partition_size);
    const int part = decode_partition(item.slot, np, p.np_slots);
    if (part < 0) return;
    const int G = p.num_q_heads / p.num_kv_heads;
    const int h0 = kvh * G;
    const float qnan = __builtin_nanf("");
    if (bad_len) {
        for (int i = lane; i < G * D; i += 64)
            p.out[((int64_t)s * p.num_q_heads + h0) * D + i] = qnan;
        return;
    }

    __shared__ float q_s[kMaxGroup][D];
    __shared__ float score_s[kMaxGroup][16];
    const T *q = reinterpret_cast<const T *>(p.q) + ((int64_t)s * p.num_q_heads + h0) * D;
    for (int i = lane * VEC; i < G * D; i += 64 * VEC) {
        float tmp[VEC];
        widen16<T>(q + i, tmp);
#pragma unroll
        for (int e = 0; e < VEC; ++e) q_s[(i + e) / D][(i + e) % D] = tmp[e];
    }
    __syncthreads();

    const T *kc = reinterpret_cast<const T *>(p.k_cache);
    const T *vc = reinterpret_cast<const T *>(p.v_cache);
    const int32_t *table = p.block_tables + (int64_t)s * p.table_stride;
    const int32_t t_begin = part * p.partition_size;
    const int32_t t_end = min(L, t_begin + p.partition_size);

    float m[kMaxGroup], l[kMaxGroup], acc[kMaxGroup][DPL];
    for (int gi = 0; gi < G; ++gi) {
        m[gi] = kNegInf;
        l[gi] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[gi][e] = 0.f;
    }
    bool bad_block = false;

    for (int32_t t0 = t_begin; t0 < t_end; t0 += 16) {
        int32_t bid = table[t0 / BS];
        if ((uint32_t)bid >= (uint32_t)p.num_blocks) {
            bad_block = true;
            bid = 0;
        }
        const int off = t0 % BS;
        const int64_t bh = (int64_t)bid * p.num_kv_heads + kvh;
        // q.k for token t0 + r (rows past L stay inside this allocated block).
        float kr[QD];
        const T *krow = kc + (bh * BS + off + r) * D + c * QD;
#pragma unroll
        for (int i = 0; i < QD; i += VEC) widen16<T>(krow + i, kr + i);
        const bool valid = t0 + r < L;
        for (int gi = 0; gi < G; ++gi) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < QD; ++i) dot += q_s[gi][c * QD + i] * kr[i];
            dot = group_sum<4>(dot);
            if (c == 0) score_s[gi][r] = valid ? dot * p.scale_log2 : kNegInf;
        }
        __syncthreads();
        // P V for this lane's dims over the step's valid tokens.
        const int nvalid = min(16, L - t0);
        float vrow[DPL][16];
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const T *vp = vc + (bh * D + lane + 64 * e) * BS + off;
#pragma unroll
            for (int i = 0; i < 16; i += VEC) widen16<T>(vp + i, vrow[e] + i);
        }
        for (int gi = 0; gi < G; ++gi) {
            float mx = kNegInf;
            for (int t = 0; t < 16; ++t) mx = fmaxf(mx, score_s[gi][t]);
            const float m_new = fmaxf(m[gi], mx);
            const float f = exp2f(m[gi] - m_new);
            l[gi] *= f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[gi][e] *= f;
            for (int t = 0; t < nvalid; ++t) {
                const float pt = exp2f(score_s[gi][t] - m_new);
                l[gi] += pt;
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[gi][e] += pt * vrow[e][t];
            }
            m[gi] = m_new;
        }
        __syncthreads();
    }

    for (int gi = 0; gi < G; ++gi) {
        const int h = h0 + gi;
        if (np == 1) {
            const float inv = l[gi] > 0.f ? 1.f / l[gi] : 0.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                p.out[((int64_t)s * p.num_q_heads + h) * D + lane + 64 * e] =
                    bad_block ? qnan : acc[gi][e] * inv;
        } else {
            const int64_t slot = ((int64_t)s * p.num_q_heads + h) * p.np_slots + part;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                p.ws_o[slot * D + lane + 64 * e] = bad_block ? qnan : acc[gi][e];
            if (lane == 0) {
                p.ws_ml[2 * slot] = bad_block ? qnan : m[gi];
                p.ws_ml[2 * slot + 1] = bad_block ? qnan : l[gi];
            }
        }
    }
}

}  // namespace

int launch_decode_valu(const DecodeParams &p, pa_dtype dtype, void *stream) {
    if (p.num_seqs == 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)((int64_t)p.np_slots * p.num_kv_heads * p.num_seqs));
    if (dtype == PA_DTYPE_F32) {
        if (p.head_dim == 64)
            hipLaunchKernelGGL((decode_valu_kernel<uint32_t, 64>), grid, dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((decode_valu_kernel<uint32_t, 128>), grid, dim3(64), 0, s, p);
    } else {
        if (p.head_dim == 64)
            hipLaunchKernelGGL((decode_valu_kernel<uint16_t, 64>), grid, dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((decode_valu_kernel<uint16_t, 128>), grid, dim3(64), 0, s, p);
    }
    return (int)hipGetLastError();
}

}  // namespace pa
