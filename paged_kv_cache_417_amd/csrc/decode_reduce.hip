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
constexpr int kReduceChunk = 1024;  // partitions whose weights sit in LDS at once

// Max (or sum) over the 256 threads of the workgroup; every thread gets it.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float *scratch) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const float o = xor_shuffle(v, m);
        v = MAX ? fmaxf(v, o) : v + o;
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // scratch free from any earlier use
    if ((threadIdx.x & 63) == 0) scratch[wave] = v;
    __syncthreads();
    float r = scratch[0];
#pragma unroll
    for (int i = 1; i < kReduceThreads / 64; ++i) r = MAX ? fmaxf(r, scratch[i]) : r + scratch[i];
    return r;
}

// One workgroup of 256 threads per (sequence, query head).  The partitions'
// maxima are read in parallel and reduced; each thread then owns one dim d
// and one slice of the partitions (256 / D slices), summing its weighted
// partial outputs with independent loads; the slices are added in LDS.  The
// order of every sum depends only on partition indices: deterministic.
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeParams p) {
    __shared__ float w_s[kReduceChunk];
    __shared__ float o_s[kReduceThreads];
    __shared__ float scratch[kReduceThreads / 64];
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

    float mx = kNegInf;
    for (int32_t i = tid; i < np; i += kReduceThreads) mx = fmaxf(mx, ml[2 * i]);
    const float M = block_reduce<true>(mx, scratch);

    const int D = p.head_dim;
    const int slices = kReduceThreads / D;
    const int d = tid % D, sl = tid / D;
    float lpart = 0.f, o = 0.f;
    for (int32_t c0 = 0; c0 < np; c0 += kReduceChunk) {
        const int32_t cn = min(kReduceChunk, np - c0);
        for (int32_t i = tid; i < cn; i += kReduceThreads) {
            const float w = fast_exp2(ml[2 * (c0 + i)] - M);
            w_s[i] = w;
            lpart += w * ml[2 * (c0 + i) + 1];
        }
        __syncthreads();
        const float *op = p.ws_o + (base + c0) * D + d;
#pragma unroll 8
        for (int32_t i = sl; i < cn; i += slices) o += w_s[i] * op[(int64_t)i * D];
        __syncthreads();
    }
    const float lsum = block_reduce<false>(lpart, scratch);
    o_s[tid] = o;
    __syncthreads();
    if (tid < D) {
        float t = o_s[tid];
        for (int k = 1; k < slices; ++k) t += o_s[k * D + tid];
        p.out[((int64_t)s * p.num_q_heads + h) * D + tid] = t / lsum;
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
