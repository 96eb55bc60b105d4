// decode_mfma.hip — paged decode attention for bf16 KV on the gfx950 matrix
// cores, one wave per (sequence, kv head, partition).
//
// Sources (page title, section):
//   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1 — the kernel finds every
//        physical block of a sequence through its block table and reads K/V
//        from those scattered blocks; §3.3 — scaling, softmax and weighted sum
//        fused in one kernel, access pattern built for memory bandwidth.
//   [VF] 《大模型推理：vLLM大模型推理框架（附下载）》 §1.1 — segments of one
//        sequence can be processed independently (split-K partitions).
//
// Work split.  The wave walks its partition in steps of 32 tokens.  All G
// query heads of the kv head ride in the 16 columns of one MFMA tile, so K
// and V are read once per group; for MHA only column 0 is live.  The tile is
// wasteful in flops (G/16 of it is used) but decode moves one byte per flop
// or so: the bound is HBM, and the matrix core removes the per-token
// cross-lane dot-product reductions the vector ALU would need.
//
// Per step (lane = 16*g + n, g in 0..3, n in 0..15):
//   S = K q^T : two v_mfma_f32_16x16x32_bf16 chains (tiles a and b), A = K
//       rows, B = q columns.  Tile a's A row n is token 8*(n/4) + n%4, tile
//       b's is that + 4, so afterwards lane (g, n) holds the scores of tokens
//       8g .. 8g+7 of head n -- exactly the B operand layout PV needs.  Head
//       dims are assigned to MFMA k-slots as d = 64*(ks/2) + 16*g + 8*(ks%2)
//       + i for A and B alike, so each lane reads 32 contiguous bytes per
//       64-dim slab.
//   online softmax : running max shared by the four lanes of a head (two
//       butterfly exchanges), per-lane running sum; exp2 with log2(e) folded
//       into the scale.
//   O += P V : A = V^T rows (dimension-major V layout gives 8 consecutive
//       tokens per lane in one 16-byte load), B = P.  P is fed as a bf16 hi
//       part plus a bf16 remainder (two MFMAs), which keeps P's error near
//       2^-16 instead of bf16's 2^-9.
// Tokens at or past the context length are excluded by selecting -inf
// scores and zero V elements (NaN-poisoned rows cannot leak), and their
// addresses are clamped onto the last valid token so no unallocated block is
// touched.
//
// fp8 cache (OCP E4M3 codes, one scale per cache).  The same walk reads half
// the bytes: a lane's 16 K dims of a token are one 16-byte load, its 8 V
// tokens of a dim one 8-byte load.  Codes become bf16 exactly in registers
// (e4m3x8_to_bf16x8) and feed the same MFMAs; the K scale is folded into the
// score scale and the V scale into the output, both in fp32.
#include <type_traits>

#include "decode_split.h"
#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

template <int D>
struct StepRegs {
    u32x4 ka[D / 32];  // K rows for tile a, one 16-byte k-slot per MFMA k-step
    u32x4 kb[D / 32];
    u32x4 vt[D / 16];  // V^T rows d = 16*j + n, 8 tokens each
};

template <int D, int BS, bool TAIL, bool NT>
__device__ __forceinline__ void load_step(StepRegs<D> &r, const uint16_t *__restrict__ kc,
                                          const uint16_t *__restrict__ vc, int32_t t0, int32_t L,
                                          int32_t bidA, int32_t bidB, int32_t hkv, int32_t kvh,
                                          int lane) {
    const int n = lane & 15, g = lane >> 4;
    int ta = t0 + 8 * (n >> 2) + (n & 3);
    int tb = ta + 4;
    int tv = t0 + 8 * g;
    if (TAIL) {
        ta = min(ta, L - 1);
        tb = min(tb, L - 1);
        tv = min(tv, (L - 1) & ~7);
    }
    // Within a 32-token step the tokens span one block (BS >= 32) or two
    // consecutive ones (BS == 16): the second holds step tokens 16..31.
    const int32_t ba = (BS == 16 && ta - t0 >= 16) ? bidB : bidA;
    const int32_t bb = (BS == 16 && tb - t0 >= 16) ? bidB : bidA;
    const int32_t bv = (BS == 16 && tv - t0 >= 16) ? bidB : bidA;
    const uint16_t *ka = kc + (((int64_t)ba * hkv + kvh) * BS + (ta % BS)) * D;
    const uint16_t *kb = kc + (((int64_t)bb * hkv + kvh) * BS + (tb % BS)) * D;
    const uint16_t *vp = vc + (((int64_t)bv * hkv + kvh) * D + n) * BS + (tv % BS);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        r.ka[ks] = NT ? ld16_nt(ka + kslot_dim(ks, g)) : ld16(ka + kslot_dim(ks, g));
        r.kb[ks] = NT ? ld16_nt(kb + kslot_dim(ks, g)) : ld16(kb + kslot_dim(ks, g));
    }
    // A step reads whole V^T rows of a block when BS <= 32; with larger
    // blocks it reads 64 of each row's 2*BS bytes and the following steps
    // read the rest of those cache lines, so the lines must stay cached.
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
        r.vt[j] = NT && BS <= 32 ? ld16_nt(vp + (int64_t)j * 16 * BS)
                                 : ld16(vp + (int64_t)j * 16 * BS);
}

// fp8 step registers: K codes of tiles a and b (16 dims per 16-byte load:
// k-slots 2p and 2p+1), V codes (8 tokens of one dim per 8-byte load).
template <int D>
struct StepRaw8 {
    u32x4 k[2][D / 64];
    u32x2 vt[D / 16];
};

template <int D, int BS, bool TAIL, bool NT>
__device__ __forceinline__ void load_step_fp8(StepRaw8<D> &r, const uint8_t *__restrict__ kc,
                                              const uint8_t *__restrict__ vc, int32_t t0,
                                              int32_t L, int32_t bidA, int32_t bidB, int32_t hkv,
                                              int32_t kvh, int lane) {
    const int n = lane & 15, g = lane >> 4;
    int ta = t0 + 8 * (n >> 2) + (n & 3);
    int tb = ta + 4;
    int tv = t0 + 8 * g;
    if (TAIL) {
        ta = min(ta, L - 1);
        tb = min(tb, L - 1);
        tv = min(tv, (L - 1) & ~7);
    }
    const int32_t ba = (BS == 16 && ta - t0 >= 16) ? bidB : bidA;
    const int32_t bb = (BS == 16 && tb - t0 >= 16) ? bidB : bidA;
    const int32_t bv = (BS == 16 && tv - t0 >= 16) ? bidB : bidA;
    const uint8_t *ka = kc + (((int64_t)ba * hkv + kvh) * BS + (ta % BS)) * D + 16 * g;
    const uint8_t *kb = kc + (((int64_t)bb * hkv + kvh) * BS + (tb % BS)) * D + 16 * g;
    const uint8_t *vp = vc + (((int64_t)bv * hkv + kvh) * D + n) * BS + (tv % BS);
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
        r.k[0][c] = NT ? ld16_nt(ka + 64 * c) : ld16(ka + 64 * c);
        r.k[1][c] = NT ? ld16_nt(kb + 64 * c) : ld16(kb + 64 * c);
    }
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
        r.vt[j] = NT && BS <= 32 ? ld8_nt(vp + (int64_t)j * 16 * BS) : ld8(vp + (int64_t)j * 16 * BS);
}

// fp8 codes -> the bf16 step registers compute_step takes (exact).
template <int D>
__device__ __forceinline__ void widen_step(const StepRaw8<D> &r, StepRegs<D> &o) {
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
        o.ka[2 * c] = e4m3x8_to_bf16x8(u32x2{r.k[0][c][0], r.k[0][c][1]});
        o.ka[2 * c + 1] = e4m3x8_to_bf16x8(u32x2{r.k[0][c][2], r.k[0][c][3]});
        o.kb[2 * c] = e4m3x8_to_bf16x8(u32x2{r.k[1][c][0], r.k[1][c][1]});
        o.kb[2 * c + 1] = e4m3x8_to_bf16x8(u32x2{r.k[1][c][2], r.k[1][c][3]});
    }
#pragma unroll
    for (int j = 0; j < D / 16; ++j) o.vt[j] = e4m3x8_to_bf16x8(r.vt[j]);
}

template <int D, bool TAIL>
__device__ __forceinline__ void compute_step(const StepRegs<D> &r, const bf16x8 *qb, int32_t t0,
                                             int32_t L, float scale_log2, float &m, float &l,
                                             floatx4 *acc, int lane) {
    const int g = lane >> 4;
    floatx4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.ka[ks]), qb[ks], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.kb[ks]), qb[ks], sb, 0, 0, 0);
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        z[i] = sa[i] * scale_log2;
        z[4 + i] = sb[i] * scale_log2;
    }
    const int tbase = t0 + 8 * g;
    if (TAIL) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (tbase + i >= L) z[i] = kNegInf;
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = rows4_max(mx);
    const float m_new = fmaxf(m, mx);
    const float f = fast_exp2(m - m_new);
    float p[8], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = fast_exp2(z[i] - m_new);
        sum += p[i];
    }
    l = l * f + sum;
    m = m_new;
    bf16x8 ph, pl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 hi = (__bf16)p[i];
        ph[i] = hi;
        pl[i] = (__bf16)(p[i] - (float)hi);
    }
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
        acc[j] *= f;
        u32x4 v = r.vt[j];
        if (TAIL) {
            // zero the bf16 elements of tokens >= L (pairs packed per dword)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int t = tbase + 2 * w;
                uint32_t keep = (t < L ? 0x0000ffffu : 0u) | (t + 1 < L ? 0xffff0000u : 0u);
                v[w] &= keep;
            }
        }
        const bf16x8 vb = as_bf16x8(v);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, ph, acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pl, acc[j], 0, 0, 0);
    }
}

// The walk over partition `part` of sequence s (np partitions in all),
// tokens [t_begin, t_end), for kv head kvh, or its NaN rows when the length
// is bad.  Only the sequence's last partition may end off a 32-token step,
// at its context length t_end.
template <int D, int BS, bool NT, bool FP8>
__device__ __forceinline__ void decode_part(const DecodeParams &p, int kvh, int s, int part,
                                            int32_t t_begin, int32_t t_end, int32_t np,
                                            bool bad_len) {
    using Regs = std::conditional_t<FP8, StepRaw8<D>, StepRegs<D>>;
    const int lane = threadIdx.x;
    const int n = lane & 15, g = lane >> 4;
    const int G = p.num_q_heads / p.num_kv_heads;
    const int h = kvh * G + n;  // this lane's query head (live when n < G)
    const bool live = n < G;
    float *out_row = p.out + ((int64_t)s * p.num_q_heads + h) * D;

    if (bad_len) {
        if (live) {
            const floatx4 nan4 = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                  __builtin_nanf("")};
#pragma unroll
            for (int j = 0; j < D / 16; ++j)
                *reinterpret_cast<floatx4 *>(out_row + 16 * j + 4 * g) = nan4;
        }
        return;
    }

    // q as the B operand: column n = head, k-slot dims per kslot_dim().
    bf16x8 qb[D / 32];
    const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                           ((int64_t)s * p.num_q_heads + (live ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        u32x4 v = ld16(qrow + kslot_dim(ks, g));
        if (!live) v = u32x4{0u, 0u, 0u, 0u};
        qb[ks] = as_bf16x8(v);
    }

    const uint16_t *kc = reinterpret_cast<const uint16_t *>(p.k_cache);
    const uint16_t *vc = reinterpret_cast<const uint16_t *>(p.v_cache);
    const int32_t *table = p.block_tables + (int64_t)s * p.table_stride;
    const int32_t L = t_end;  // tokens at or past it are masked (last step only)
    const int32_t nsteps = (t_end - t_begin + 31) / 32;
    const bool has_tail = ((t_end - t_begin) & 31) != 0;

    float m = kNegInf, lsum = 0.f;
    floatx4 acc[D / 16];
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // The partition's block-table slice lives in one VGPR (lane j holds the
    // entry of logical block win + j); block ids are read with readlane, so
    // no table load sits between a step's issue and the previous step's data.
    const int32_t b_last = (t_end - 1) / BS;  // last logical block of the partition
    int32_t win = t_begin / BS;
    int32_t tbl = (nsteps > 0 && win + lane <= b_last) ? table[win + lane] : 0;
    bool bad_block = false;
    auto block_id = [&](int32_t j) -> int32_t {
        if (j - win >= 64) {  // next 64 entries (partitions longer than 64 blocks)
            win = j;
            tbl = (win + lane <= b_last) ? table[win + lane] : 0;
            // Wait here, on this rare path only (vmcnt(0)): the window is
            // then never pending where the paths join, so the readlane below
            // does not wait for the step loads in flight.
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        int32_t b = __builtin_amdgcn_readlane(tbl, j - win);
        if ((uint32_t)b >= (uint32_t)p.num_blocks) {
            bad_block = true;
            b = 0;
        }
        return b;
    };
    // Step s covers tokens t_begin + 32 s .. +31.  Loads clamp past the end
    // of the context (a no-op except in the tail step), compute masks there.
    auto issue = [&](Regs &r, int32_t st) {
        const int32_t t0 = t_begin + 32 * st;
        const int32_t bA = block_id(t0 / BS);
        const int32_t bB = BS == 16 ? block_id(min((t0 + 16) / BS, b_last)) : bA;
        if constexpr (FP8)
            load_step_fp8<D, BS, true, NT>(r, reinterpret_cast<const uint8_t *>(p.k_cache),
                                           reinterpret_cast<const uint8_t *>(p.v_cache), t0, L,
                                           bA, bB, p.num_kv_heads, kvh, lane);
        else
            load_step<D, BS, true, NT>(r, kc, vc, t0, L, bA, bB, p.num_kv_heads, kvh, lane);
    };
    auto consume = [&](const Regs &raw, int32_t st) {
        const int32_t t0 = t_begin + 32 * st;
        const StepRegs<D> *rp;
        StepRegs<D> wide;
        if constexpr (FP8) {
            widen_step<D>(raw, wide);
            rp = &wide;
        } else {
            rp = &raw;
        }
        if (has_tail && st == nsteps - 1)
            compute_step<D, true>(*rp, qb, t0, L, p.scale_log2, m, lsum, acc, lane);
        else
            compute_step<D, false>(*rp, qb, t0, L, p.scale_log2, m, lsum, acc, lane);
    };

    // Two register buffers in ping-pong: while one step is consumed the next
    // one's loads are in flight.  No buffer is ever copied into the other.
    // The second issue of the body is conditional, so after it the compiler
    // waits for every load before the next step's math: each step still
    // overlaps the other buffer's loads, and no load is ever issued twice.
    // (An unconditional issue clamped to the last step keeps two steps in
    // flight throughout, but its one re-read per partition reaches HBM: 5%
    // more traffic and 5% slower on the 7B-shaped batch, which already
    // streams at about 90% of a plain copy's read rate.)
    if (nsteps > 0) {
        Regs ra, rb;
        issue(ra, 0);
        int32_t st = 0;
        for (; st + 1 < nsteps; st += 2) {
            issue(rb, st + 1);
            consume(ra, st);
            if (st + 2 < nsteps) issue(ra, st + 2);
            consume(rb, st + 1);
        }
        if (st < nsteps) consume(ra, st);
    }

    lsum = rows4_sum(lsum);
    if (!live) return;
    const float qnan = __builtin_nanf("");
    // An fp8 cache's V scale multiplies the output (1 for bf16).
    const float vs = FP8 ? p.v_scale : 1.f;
    if (np == 1) {
        const float inv = lsum > 0.f ? vs / lsum : 0.f;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            floatx4 o = acc[j] * inv;
            if (bad_block) o = floatx4{qnan, qnan, qnan, qnan};
            *reinterpret_cast<floatx4 *>(out_row + 16 * j + 4 * g) = o;
        }
    } else {
        const int64_t slot = ((int64_t)s * p.num_q_heads + h) * p.np_slots + part;
        float *o_part = p.ws_o + slot * D;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            floatx4 o = FP8 ? acc[j] * vs : acc[j];
            if (bad_block) o = floatx4{qnan, qnan, qnan, qnan};
            *reinterpret_cast<floatx4 *>(o_part + 16 * j + 4 * g) = o;
        }
        if (g == 0) {
            p.ws_ml[2 * slot] = bad_block ? qnan : m;
            p.ws_ml[2 * slot + 1] = bad_block ? qnan : lsum;
        }
    }
}


// One per-sequence work item of the slot grid: (kv head, sequence,
// partition slot) of the 1-D grid index.  GROUPED: a grouped call, whose
// shared partitions are the group kernel's and whose members' private
// partitions start at the end of their group's shared region.
template <int D, int BS, bool NT, bool FP8, bool GROUPED>
__device__ __forceinline__ void decode_seq_item(const DecodeParams &p, uint32_t index) {
    const DecodeItem item = decode_item(index, p.num_kv_heads, p.num_seqs);
    const int32_t L = p.context_lens[item.seq];
    const int32_t gid = GROUPED ? p.seq_group[item.seq] : -1;  // loaded beside L
    const bool bad_len = bad_length(p, L, BS);
    const SeqSplit sp = GROUPED ? seq_split(p, item.seq, gid, L, bad_len)
                                : SeqSplit{num_parts(p, L, bad_len), 0, 0};
    const int part = decode_partition(item.slot, sp.np, p.np_slots);
    if (part < sp.shared) return;  // no partition in this slot, or the group's
    const int32_t t_begin = sp.t_shared + (part - sp.shared) * p.partition_size;
    const int32_t t_end = bad_len ? t_begin : min(L, t_begin + p.partition_size);
    decode_part<D, BS, NT, FP8>(p, item.kvh, item.seq, part, t_begin, t_end, sp.np, bad_len);
}

// Shared partitions of a group of sequences, one wave per (kv head, group,
// member chunk, partition).  Partition i of the group's shared region (T
// tokens) is [i ps, min((i + 1) ps, T)); the wave reads its K/V once, through
// the leader's block table, and serves 16 / G members at once: MFMA column n
// is member n / G of the chunk, query head n % G of the kv head (the same
// layout the per-sequence kernel gives the G heads of one sequence), so each
// member's partial is the one the per-sequence walk of that token range
// gives.  Members whose context ends at or before T are not served (they
// are decoded alone, member_shares()).  A member whose own table differs
// from the leader's over the partition gets NaN partials (its row comes out
// NaN); a bad block id makes every member's partials NaN.
template <int D, int BS, bool NT, bool FP8>
__device__ __forceinline__ void decode_group_item(const DecodeParams &p, uint32_t item) {
    using Regs = std::conditional_t<FP8, StepRaw8<D>, StepRegs<D>>;
    const uint32_t r1 = item / (uint32_t)p.num_kv_heads;
    const int kvh = (int)(item - r1 * (uint32_t)p.num_kv_heads);
    const uint32_t r2 = r1 / (uint32_t)p.num_groups;
    const int grp = (int)(r1 - r2 * (uint32_t)p.num_groups);
    const int part = (int)(r2 / (uint32_t)p.grp_chunks);
    const int chunk = (int)(r2 - (uint32_t)part * (uint32_t)p.grp_chunks);
    const int lane = threadIdx.x;
    const int n = lane & 15, g = lane >> 4;

    // The group's run and shared partitions (scalar loads, issued together).
    // A wave starts streaming after only these and one round of vector
    // loads: every load that decides which columns are live, and the
    // members' table slices, go out in that one round.
    const int32_t lo = p.grp_offsets[grp], hi = p.grp_offsets[grp + 1];
    const int64_t T = shared_tokens(p, p.grp_shared[grp]);
    if (lo < 0 || lo >= p.num_seqs) return;
    const int G = p.num_q_heads / p.num_kv_heads;
    const int mpw = 16 / G;  // members per wave
    // No member is live unless the partition starts inside the shared region
    // and the chunk's first member lies in the group's run.
    if ((int64_t)part * p.partition_size >= T || lo + chunk * mpw >= hi) return;
    // this lane's column: member s_n, query head h
    const int32_t s_n = lo + chunk * mpw + n / G;
    const int h = kvh * G + n % G;
    const bool in_range = n < mpw * G && s_n < p.num_seqs;

    const uint16_t *kc = reinterpret_cast<const uint16_t *>(p.k_cache);
    const uint16_t *vc = reinterpret_cast<const uint16_t *>(p.v_cache);
    const int32_t *table = p.block_tables + (int64_t)lo * p.table_stride;
    // A shared partition lies wholly inside every live member's context
    // (T < L_n); only the region's last one may end off a 32-token step.
    const int32_t t_begin = part * p.partition_size;
    const int32_t t_end = (int32_t)min((int64_t)t_begin + p.partition_size, T);
    const int32_t L = t_end;  // tokens at or past it are masked
    const int32_t nsteps = (t_end - t_begin + 31) / 32;
    const bool has_tail = ((t_end - t_begin) & 31) != 0;
    const int32_t b_first = t_begin / BS, b_last = (t_end - 1) / BS;

    // one round of loads: the member's group and length, q, the leader's
    // first table window, the members' first table windows
    const int32_t s_col = in_range ? s_n : lo;
    const int32_t grp_of = p.seq_group[s_col];
    const int32_t L_n = p.context_lens[s_col];
    bf16x8 qb[D / 32];
    const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                           ((int64_t)s_col * p.num_q_heads + (in_range ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qb[ks] = as_bf16x8(ld16(qrow + kslot_dim(ks, g)));
    // (these loads precede the liveness check, which is what bounds b_last
    // by a member's table for a well-formed group: clamp to the row too)
    const int32_t jw = b_first + lane;  // this lane's entry of the first window
    const bool jw_in = jw <= b_last && jw < p.table_stride;
    int32_t tbl = jw_in ? table[jw] : 0;
    int32_t mt[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int32_t s_k = lo + chunk * mpw + k;
        mt[k] = (k < mpw && s_k < p.num_seqs && jw_in)
                    ? p.block_tables[(int64_t)s_k * p.table_stride + jw]
                    : 0;
    }

    // a column is live when its sequence belongs to this group's run and
    // its context extends past the shared region: member_shares(), the test
    // the per-sequence items and the merge apply
    const bool live = in_range && grp_of == grp &&
                      member_shares(p, s_n, grp_of, lo, hi, T, L_n, bad_length(p, L_n, BS));
    if (!__any(live)) return;
    if (!live) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) qb[ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }

    // Each live member's table must equal the leader's over the partition:
    // the first 64 entries from the loads above, any further ones 64 at a
    // time, member by member.
    bool bad_table = false;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (k >= mpw || !__shfl(live ? 1 : 0, k * G, 64)) continue;  // column k * G is member k
        bool diff = jw_in && mt[k] != tbl;
        const int32_t *mtk = p.block_tables + (int64_t)(lo + chunk * mpw + k) * p.table_stride;
        for (int32_t b = b_first + 64; b <= b_last; b += 64) {
            const int32_t jj = b + lane;
            diff = diff || (jj <= b_last && mtk[jj] != table[jj]);
        }
        if (__any(diff) && n / G == k) bad_table = true;
    }

    float m = kNegInf, lsum = 0.f;
    floatx4 acc[D / 16];
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

    int32_t win = b_first;
    bool bad_block = false;
    auto block_id = [&](int32_t j) -> int32_t {
        if (j - win >= 64) {
            win = j;
            tbl = (win + lane <= b_last) ? table[win + lane] : 0;
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), on this rare path only
        }
        int32_t b = __builtin_amdgcn_readlane(tbl, j - win);
        if ((uint32_t)b >= (uint32_t)p.num_blocks) {
            bad_block = true;
            b = 0;
        }
        return b;
    };
    auto issue = [&](Regs &r, int32_t st) {
        const int32_t t0 = t_begin + 32 * st;
        const int32_t bA = block_id(t0 / BS);
        const int32_t bB = BS == 16 ? block_id(min((t0 + 16) / BS, b_last)) : bA;
        if constexpr (FP8)
            load_step_fp8<D, BS, true, NT>(r, reinterpret_cast<const uint8_t *>(p.k_cache),
                                           reinterpret_cast<const uint8_t *>(p.v_cache), t0, L,
                                           bA, bB, p.num_kv_heads, kvh, lane);
        else
            load_step<D, BS, true, NT>(r, kc, vc, t0, L, bA, bB, p.num_kv_heads, kvh, lane);
    };
    auto consume = [&](const Regs &raw, int32_t st) {
        const int32_t t0 = t_begin + 32 * st;
        const StepRegs<D> *rp;
        StepRegs<D> wide;
        if constexpr (FP8) {
            widen_step<D>(raw, wide);
            rp = &wide;
        } else {
            rp = &raw;
        }
        if (has_tail && st == nsteps - 1)
            compute_step<D, true>(*rp, qb, t0, L, p.scale_log2, m, lsum, acc, lane);
        else
            compute_step<D, false>(*rp, qb, t0, L, p.scale_log2, m, lsum, acc, lane);
    };
    // the same ping-pong as the per-sequence kernel
    {
        Regs ra, rb;
        issue(ra, 0);
        int32_t st = 0;
        for (; st + 1 < nsteps; st += 2) {
            issue(rb, st + 1);
            consume(ra, st);
            if (st + 2 < nsteps) issue(ra, st + 2);
            consume(rb, st + 1);
        }
        if (st < nsteps) consume(ra, st);
    }

    lsum = rows4_sum(lsum);
    if (!live) return;
    const float qnan = __builtin_nanf("");
    const float vs = FP8 ? p.v_scale : 1.f;
    const bool bad = bad_block || bad_table;
    const int64_t slot = ((int64_t)s_n * p.num_q_heads + h) * p.np_slots + part;
    float *o_part = p.ws_o + slot * D;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
        floatx4 o = FP8 ? acc[j] * vs : acc[j];
        if (bad) o = floatx4{qnan, qnan, qnan, qnan};
        *reinterpret_cast<floatx4 *>(o_part + 16 * j + 4 * g) = o;
    }
    if (g == 0) {
        p.ws_ml[2 * slot] = bad ? qnan : m;
        p.ws_ml[2 * slot + 1] = bad ? qnan : lsum;
    }
}

// Two waves per SIMD: the two step buffers (64 VGPRs each at D = 128) fit
// in 256 registers without spills.  FP8: the cache holds E4M3 codes.
template <int D, int BS, bool NT, bool FP8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_mfma_kernel(
    DecodeParams p) {
    decode_seq_item<D, BS, NT, FP8, false>(p, blockIdx.x);
}

// Grouped decode in one grid: the first group_items workgroups compute the
// groups' shared partitions, the rest are the per-sequence items (which skip
// those partitions).  One launch, so the shared partitions' waves and the
// per-sequence ones fill the chip together instead of draining in turn.
template <int D, int BS, bool NT, bool FP8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_grouped_kernel(
    DecodeParams p, uint32_t group_items) {
    if (blockIdx.x < group_items)
        decode_group_item<D, BS, NT, FP8>(p, blockIdx.x);
    else
        decode_seq_item<D, BS, NT, FP8, true>(p, blockIdx.x - group_items);
}

// ---------------------------------------------------------------------------
// Longest-first decode for batches of up to kScanMaxSeqs sequences.  The
// slot grid above dispatches (kv head, sequence, slot) in slot order and
// launches a wave for every slot up to the longest sequence's partition
// count, so a batch of mixed lengths launches many waves that find no
// partition, and its last partitions (of every length) drain in sequence
// order.  Here each wave loads all the context lengths (one vector load per
// 64 sequences, in place of the slot grid's single length load) and finds
// its work item among the batch's partitions taken in this order: the bad
// lengths (a NaN row), then the full partitions (every sequence's first,
// then every second, ...), then the last, partial partitions from the
// longest to the shortest (ties in sequence order).  Waves past the last
// item exit at once, after every item's wave has been dispatched, and the
// grid drains with its shortest partitions.  Every partition is computed
// exactly as in the slot grid.
constexpr int kScanMaxSeqs = 256;

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}
__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__builtin_popcountll(m); }
// the lane holding the r-th set bit of m (r < popcount(m))
__device__ __forceinline__ int nth_set_lane(uint64_t m, uint32_t r, int lane) {
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const bool mine = ((m >> lane) & 1ull) != 0 && below == r;
    return __builtin_ctzll(__ballot(mine));
}

// C: chunks of 64 sequences (num_seqs <= 64 C).
template <int D, int BS, bool NT, bool FP8, int C>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_scan_kernel(
    DecodeParams p) {
    const int lane = threadIdx.x;
    const uint32_t hkv = (uint32_t)p.num_kv_heads;
    const uint32_t e0 = blockIdx.x / hkv;
    const int kvh = (int)(blockIdx.x - e0 * hkv);
    const int32_t ps = p.partition_size;
    // per lane: sequences lane, lane + 64, ...
    int32_t Lc[C], full[C], tail[C];
    bool badc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int sq = 64 * c + lane;
        const bool valid = sq < p.num_seqs;
        const int32_t L = valid ? p.context_lens[sq] : 0;
        const bool bad = valid && bad_length(p, L, BS);
        const int32_t np = num_parts(p, L, bad);
        const int32_t last = L - (np - 1) * ps;  // tokens of the last partition
        const bool ok = valid && !bad;
        Lc[c] = L;
        badc[c] = bad;
        full[c] = ok ? np - 1 + (last == ps ? 1 : 0) : 0;
        tail[c] = ok && last != ps ? (last + 31) / 32 : -1;
    }
    uint32_t nbad = 0, ntail = 0;
    int32_t nfull = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        nbad += popc64(__ballot(badc[c]));
        ntail += popc64(__ballot(tail[c] >= 0));
        nfull += wave_sum(full[c]);
    }
    uint32_t e = e0;
    if (e >= nbad + (uint32_t)nfull + ntail) return;  // no item left for this wave
    // the e-th set bit over the chunks' masks -> sequence, its length
    int s = 0;
    int32_t L = 0;
    auto pick = [&](const uint64_t *m, uint32_t r) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const uint32_t cnt = popc64(m[c]);
            if (r < cnt) {
                const int ln = nth_set_lane(m[c], r, lane);
                s = 64 * c + ln;
                L = __builtin_amdgcn_readlane(Lc[c], ln);
                return;
            }
            r -= cnt;
        }
    };
    uint64_t m[C];
    if (e < nbad) {
#pragma unroll
        for (int c = 0; c < C; ++c) m[c] = __ballot(badc[c]);
        pick(m, e);
        decode_part<D, BS, NT, FP8>(p, kvh, s, 0, 0, 0, 1, true);
        return;
    }
    e -= nbad;
    int part = 0;
    bool found = false;
    if (e < (uint32_t)nfull) {
        // full partitions, partition-major (k < np_max always finds it: the
        // counts of the k sum to nfull)
        for (int32_t k = 0; k < p.np_max; ++k) {
            uint32_t cnt = 0;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                m[c] = __ballot(full[c] > k);
                cnt += popc64(m[c]);
            }
            if (e < cnt) {
                pick(m, e);
                part = k;
                found = true;
                break;
            }
            e -= cnt;
        }
    } else {
        // last partial partitions, most steps first
        e -= (uint32_t)nfull;
        for (int32_t v = ps / 32; v >= 0; --v) {
            uint32_t cnt = 0;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                m[c] = __ballot(tail[c] == v);
                cnt += popc64(m[c]);
            }
            if (e < cnt) {
                pick(m, e);
                part = num_parts(p, L, false) - 1;
                found = true;
                break;
            }
            e -= cnt;
        }
    }
    if (!found) return;
    // wave-uniform by construction; say so, so that they stay in scalar registers
    s = __builtin_amdgcn_readfirstlane(s);
    part = __builtin_amdgcn_readfirstlane(part);
    L = __builtin_amdgcn_readfirstlane(L);
    const int32_t t_begin = part * p.partition_size;
    decode_part<D, BS, NT, FP8>(p, kvh, s, part, t_begin, min(L, t_begin + p.partition_size),
                                num_parts(p, L, false), false);
}

template <int D, int BS>
void launch_one(const DecodeParams &p, hipStream_t s) {
    const int64_t seq_items = (int64_t)p.np_slots * p.num_kv_heads * p.num_seqs;
    if (p.seq_group && p.num_groups > 0) {
        // shared partitions: ceil(T / ps) <= np_max for a region T shorter
        // than a member's context
        const int64_t group_items =
            (int64_t)p.np_max * p.grp_chunks * p.num_groups * p.num_kv_heads;
        const dim3 grid((unsigned)(group_items + seq_items));
#define PA_GROUPED(NTv, FP8v)                                                                     \
    hipLaunchKernelGGL((decode_grouped_kernel<D, BS, NTv, FP8v>), grid, dim3(64), 0, s, p,      \
                       (uint32_t)group_items)
        if (p.kv_fp8) {
            if (p.kv_reuse) PA_GROUPED(false, true); else PA_GROUPED(true, true);
        } else {
            if (p.kv_reuse) PA_GROUPED(false, false); else PA_GROUPED(true, false);
        }
#undef PA_GROUPED
        return;
    }
    const dim3 grid((unsigned)seq_items);
    if (p.np_max > 1 && p.num_seqs <= kScanMaxSeqs) {
#define PA_SCAN(NTv, FP8v, Cv) \
    hipLaunchKernelGGL((decode_scan_kernel<D, BS, NTv, FP8v, Cv>), grid, dim3(64), 0, s, p)
#define PA_SCAN_C(NTv, FP8v)                           \
    do {                                               \
        if (p.num_seqs <= 64) PA_SCAN(NTv, FP8v, 1);   \
        else if (p.num_seqs <= 128) PA_SCAN(NTv, FP8v, 2); \
        else PA_SCAN(NTv, FP8v, 4);                    \
    } while (0)
        if (p.kv_fp8) {
            if (p.kv_reuse) PA_SCAN_C(false, true); else PA_SCAN_C(true, true);
        } else {
            if (p.kv_reuse) PA_SCAN_C(false, false); else PA_SCAN_C(true, false);
        }
#undef PA_SCAN_C
#undef PA_SCAN
        return;
    }
    if (p.kv_fp8) {
        if (p.kv_reuse)
            hipLaunchKernelGGL((decode_mfma_kernel<D, BS, false, true>), grid, dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<D, BS, true, true>), grid, dim3(64), 0, s, p);
    } else if (p.kv_reuse) {
        hipLaunchKernelGGL((decode_mfma_kernel<D, BS, false, false>), grid, dim3(64), 0, s, p);
    } else {
        hipLaunchKernelGGL((decode_mfma_kernel<D, BS, true, false>), grid, dim3(64), 0, s, p);
    }
}

}  // namespace

int launch_decode_mfma(const DecodeParams &p, void *stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.num_seqs == 0) return 0;
#define PA_CASE(Dv, BSv)                                        \
    if (p.head_dim == Dv && p.block_size == BSv) {              \
        launch_one<Dv, BSv>(p, s);                              \
        return (int)hipGetLastError();                          \
    }
    PA_CASE(128, 16) PA_CASE(128, 32) PA_CASE(128, 64) PA_CASE(128, 128)
    PA_CASE(64, 16) PA_CASE(64, 32) PA_CASE(64, 64) PA_CASE(64, 128)
#undef PA_CASE
    return (int)hipErrorInvalidValue;
}

}  // namespace pa
