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
// Partitions are visited in index order (token order), so the result is
// deterministic.  A grouped call's members split at their group's shared
// region (decode_split.h), so the merge looks their split up the same way.
#include "decode_split.h"
#include "device_common.h"
#include "launch.h"

namespace pa {

size_t decode_workspace_bytes(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                              int64_t np_slots) {
    if (np_slots <= 1) return 0;
    const int64_t rows = num_seqs * num_q_heads * np_slots;
    const int64_t ml = (rows * 2 * 4 + 255) / 256 * 256;
    return (size_t)(ml + rows * head_dim * 4);
}

void decode_workspace_split(void *ws, int64_t num_seqs, int64_t num_q_heads, int64_t np_slots,
                            float **ml, float **o) {
    const int64_t rows = num_seqs * num_q_heads * np_slots;
    const int64_t ml_bytes = (rows * 2 * 4 + 255) / 256 * 256;
    *ml = reinterpret_cast<float *>(ws);
    *o = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + ml_bytes);
}

namespace {

constexpr int kReduceWaves = 4;  // (sequence, query head) items per workgroup, one per wave

// One wave per (sequence, query head): lane l holds dims l*D/64 .. of the
// output and merges the partitions 0 .. np-1 in order with the same online
// rescaling the partition kernel uses (the (m, l) pair of a partition is the
// same for every lane: scalar loads).  Deterministic: one fixed order.
template <int D>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_kernel(DecodeParams p) {
    constexpr int kDpl = D / 64;  // dims per lane
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kReduceWaves + (threadIdx.x >> 6);
    if (item >= (int64_t)p.num_seqs * p.num_q_heads) return;
    const int s = (int)(item / p.num_q_heads);
    const int h = (int)(item - (int64_t)s * p.num_q_heads);
    const int32_t L = p.context_lens[s];
    const int32_t gid = p.seq_group ? p.seq_group[s] : -1;
    const bool bad_len = bad_length(p, L, p.block_size);
    if (bad_len) return;  // row already NaN
    const int32_t np = seq_split(p, s, gid, L, false).np;
    if (np <= 1) return;  // written directly by the partition kernel
    const int64_t base = ((int64_t)s * p.num_q_heads + h) * p.np_slots;
    const float *ml = p.ws_ml + 2 * base;
    const float *op = p.ws_o + base * D + kDpl * lane;

    float m = kNegInf, l = 0.f, o[kDpl];
#pragma unroll
    for (int k = 0; k < kDpl; ++k) o[k] = 0.f;
#pragma unroll 4
    for (int32_t i = 0; i < np; ++i) {
        const float mi = ml[2 * i], li = ml[2 * i + 1];
        float oi[kDpl];
        if constexpr (kDpl == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(op + (int64_t)i * D);
            oi[0] = v.x;
            oi[1] = v.y;
        } else {
            oi[0] = op[(int64_t)i * D];
        }
        const float mn = fmaxf(m, mi);
        const float a = fast_exp2(m - mn), b = fast_exp2(mi - mn);
        l = l * a + li * b;
#pragma unroll
        for (int k = 0; k < kDpl; ++k) o[k] = o[k] * a + oi[k] * b;
        m = mn;
    }
    float *orow = p.out + ((int64_t)s * p.num_q_heads + h) * D + kDpl * lane;
    if constexpr (kDpl == 2)
        *reinterpret_cast<float2 *>(orow) = float2{o[0] / l, o[1] / l};
    else
        orow[0] = o[0] / l;
}

}  // namespace

int launch_decode_reduce(const DecodeParams &p, void *stream) {
    if (p.np_slots <= 1 || p.num_seqs == 0) return 0;
    const int64_t items = (int64_t)p.num_seqs * p.num_q_heads;
    const dim3 grid((unsigned)((items + kReduceWaves - 1) / kReduceWaves)), block(64 * kReduceWaves);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.head_dim == 128)
        hipLaunchKernelGGL(decode_reduce_kernel<128>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(decode_reduce_kernel<64>, grid, block, 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace pa
