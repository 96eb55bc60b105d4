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

constexpr int kReduceThreads = 256;

// One workgroup of 256 threads per (sequence, query head).  Thread (slice
// sl, dim d) merges partitions sl, sl + slices, ... (slices = 256 / D) with
// the same online rescaling the partition kernel uses, so its loads do not
// wait on any reduction; the slices are then merged by the first D threads.
// Every merge runs in partition-index order: the result is deterministic.
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeParams p) {
    __shared__ float part_m[kReduceThreads], part_l[kReduceThreads], part_o[kReduceThreads];
    const int s = blockIdx.x / p.num_q_heads;
    const int h = blockIdx.x % p.num_q_heads;
    const int tid = threadIdx.x;
    const int32_t L = p.context_lens[s];
    const int32_t nb = (L + p.block_size - 1) / p.block_size;
    if (L < 0 || L > p.max_context_len || nb > p.table_stride) return;  // row already NaN
    const int32_t np = max(1, (L + p.partition_size - 1) / p.partition_size);
    if (np <= 1) return;  // written directly by the partition kernel
    const int64_t base = ((int64_t)s * p.num_q_heads + h) * p.np_max;
    const float *ml = p.ws_ml + 2 * base;
    const int D = p.head_dim;
    const int slices = kReduceThreads / D;
    const int d = tid % D, sl = tid / D;
    const float *op = p.ws_o + base * D + d;

    float m = kNegInf, l = 0.f, o = 0.f;
#pragma unroll 4
    for (int32_t i = sl; i < np; i += slices) {
        const float mi = ml[2 * i], li = ml[2 * i + 1], oi = op[(int64_t)i * D];
        const float mn = fmaxf(m, mi);
        const float a = fast_exp2(m - mn), b = fast_exp2(mi - mn);
        l = l * a + li * b;
        o = o * a + oi * b;
        m = mn;
    }
    part_m[tid] = m;
    part_l[tid] = l;
    part_o[tid] = o;
    __syncthreads();
    if (tid < D) {
        float M = part_m[tid];
        for (int k = 1; k < slices; ++k) M = fmaxf(M, part_m[k * D + tid]);
        float lt = 0.f, ot = 0.f;
        for (int k = 0; k < slices; ++k) {
            const float w = fast_exp2(part_m[k * D + tid] - M);
            lt += w * part_l[k * D + tid];
            ot += w * part_o[k * D + tid];
        }
        p.out[((int64_t)s * p.num_q_heads + h) * D + tid] = ot / lt;
    }
}

}  // namespace

int launch_decode_reduce(const DecodeParams &p, void *stream) {
    if (p.np_max <= 1 || p.num_seqs == 0) return 0;
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)(p.num_seqs * p.num_q_heads)),
                       dim3(kReduceThreads), 0, reinterpret_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace pa
