// decode_reduce.hip — merge of split-K decode partitions.
//
// Source: [VF] 《大模型推理：vLLM大模型推理框架（附下载）》 §1.1 — segments of a
// sequence can be processed independently; [VE] 《加速 LLM 推理：深入了解 vLLM
// 引擎》 §3.3 — softmax then weighted sum.
//
// Partition p of a row left (m_p, l_p, o_p): its running max (log2 units),
// the sum of 2^(z - m_p) over its tokens, and the matching unnormalised
// weighted sum of V rows.  With M = max_p m_p and w_p = 2^(m_p - M):
//   out = sum_p w_p o_p / sum_p w_p l_p.
// Partitions are visited in index order, so the result is deterministic.
#include "device_common.h"
#include "launch.h"

namespace pa {

size_t decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                              int64_t np_max) {
    if (np_max <= 1) return 0;
    const int64_t rows = num_seqs * num_q_heads * np_max;
    const int64_t ml = (rows * 2 * 4 + 255) / 256 * 256;
    return (size_t)(ml + rows * head_dim * 4);
}

void decode_workspace_split(void *ws, int64_t num_seqs, int64_t num_q_heads, int64_t np_max,
                            float **ml, float **o) {
    const int64_t rows = num_seqs * num_q_heads * np_max;
    const int64_t ml_bytes = (rows * 2 * 4 + 255) / 256 * 256;
    *ml = reinterpret_cast<float *>(ws);
    *o = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + ml_bytes);
}

namespace {

// One workgroup of D threads per (sequence, query head); thread = dim.
__global__ __launch_bounds__(128) void decode_reduce_kernel(DecodeParams p) {
    const int s = blockIdx.x / p.num_q_heads;
    const int h = blockIdx.x % p.num_q_heads;
    const int d = threadIdx.x;
    const int32_t L = p.context_lens[s];
    const int32_t nb = (L + p.block_size - 1) / p.block_size;
    if (L < 0 || L > p.max_context_len || nb > p.table_stride) return;  // row already NaN
    const int32_t np = max(1, (L + p.partition_size - 1) / p.partition_size);
    if (np <= 1) return;  // written directly by the partition kernel
    const int64_t base = ((int64_t)s * p.num_q_heads + h) * p.np_max;
    float M = kNegInf;
    for (int32_t i = 0; i < np; ++i) M = fmaxf(M, p.ws_ml[2 * (base + i)]);
    float lsum = 0.f, o = 0.f;
    for (int32_t i = 0; i < np; ++i) {
        const float w = exp2f(p.ws_ml[2 * (base + i)] - M);
        lsum += w * p.ws_ml[2 * (base + i) + 1];
        o += w * p.ws_o[(base + i) * p.head_dim + d];
    }
    p.out[((int64_t)s * p.num_q_heads + h) * p.head_dim + d] = o / lsum;
}

}  // namespace

int launch_decode_reduce(const DecodeParams &p, void *stream) {
    if (p.np_max <= 1 || p.num_seqs == 0) return 0;
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)(p.num_seqs * p.num_q_heads)),
                       dim3(p.head_dim), 0, reinterpret_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace pa
