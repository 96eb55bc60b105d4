// prefill.hip — chunked causal prefill over paged K/V on the gfx950 matrix
// cores (bf16 in, fp32 accumulate, fp32 out).
//
// Sources (page title, section):
//   [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §1 — one
//        iteration carries requests in different phases (prompt chunks beside
//        decode rows).
//   [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1 — K/V found through the
//        block table in scattered blocks; §3.3 — scaling, softmax, weighted
//        sum fused, matrix products on the matrix units.
//
// Work split.  One workgroup of four waves per (request, kv head, chunk of
// query positions).  The workgroup serves 128 (position, head) pairs: all G
// query heads of the kv head for 128 / G consecutive positions, so each K/V
// tile is fetched from HBM once for the whole group.  Pair c of wave w is
// w * 32 + c; head = pair % G, position = pair / G.  Each wave holds its 32
// pairs as the 16 columns of two MFMA tiles.
//
// Per 32-key step:
//   staging : the workgroup copies K [32 keys][D] and V^T [D][32 keys] of the
//       step from the paged pools into LDS (double-buffered; the next step's
//       global loads are in flight while the current step computes).  K rows
//       are stored in MFMA row order and padded by 16 bytes per row; V^T
//       rows are unpadded with their 16-byte chunks XOR-swizzled by row, so
//       that both the stage stores and the MFMA reads spread over the LDS
//       banks.
//   S^T = K Q^T : v_mfma_f32_16x16x32_bf16, A = K rows (tile a: keys
//       8*(n/4) + n%4, tile b: those + 4), B = the wave's q columns; lane
//       (g, n) ends with the scores of keys 8g .. 8g+7 of column n.
//   causal mask + online softmax : keys past a column's position get -inf
//       (a select, so no value of a masked key reaches the result); the
//       running max is shared by the four lanes of a column.
//   O^T += V^T P^T : v_mfma_f32_16x16x32_f16, A = V^T rows from LDS held as
//       fp16, B = P rounded to fp16 (relative error 2^-11, one MFMA per
//       tile).  V reaches LDS as fp16: a bf16 V element of magnitude in
//       [2^-14, 2^16) converts exactly; a smaller one lands in fp16's
//       subnormal range and keeps its bits down to 2^-24 only (an absolute
//       error under 2^-25, about 3e-8, per element); an E4M3 code always
//       converts exactly.  The weights are lifted by 2^7 before rounding
//       (they stay below 2^15) so that weights down to 2^-21 of the running
//       maximum keep full fp16 precision.
//   Exact fallback: a staged V element that fp16 cannot carry (a bf16
//       element of 2^16 or more in magnitude, an infinity or a NaN, or an
//       E4M3 NaN code) leaves a non-finite value in the accumulators of a
//       wave of the workgroup, which the end of the walk detects.  The
//       workgroup then discards its result and walks again with V in bf16
//       and P as a bf16 high part plus a bf16 remainder (two MFMAs per tile,
//       P's error near 2^-16).  In that walk non-finite V elements are staged
//       as zeros, and an output element (row, head, dim) becomes NaN exactly
//       when a key its row sees holds a non-finite V element in that dim: a
//       key past a row's position never reaches the row, as in the
//       definition.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Eight OCP E4M3 codes (bytes of w, lowest first) -> eight fp16 values, in
// order, two codes per v_cvt_scalef32_pk_f16_fp8 with scale 1.  Exact:
// every E4M3 value (at most 448 in magnitude, four significant bits, no
// smaller than 2^-9) is an fp16 value.  (The bf16 widening is
// e4m3x8_to_bf16x8.)
__device__ __forceinline__ u32x4 e4m3x8_to_f16x8(u32x2 w) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        r[2 * h] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.f, false));
        r[2 * h + 1] = __builtin_bit_cast(uint32_t,
                                          __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.f, true));
    }
    return r;
}


constexpr int kWaves = 4;
constexpr int kPairs = kWaves * 32;  // (position, head) pairs per workgroup
constexpr int kTile = 32;            // keys per step
constexpr float kRescaleMargin = 8.f;  // log2 units; weights stay below 2^8
// fp16 weights are computed as 2^kF16Lift times the true weight: below
// 2^(8 + 7) = 32768, within fp16's range, with fp16's normal range reaching
// down to 2^-21 of the running maximum.  The sum l carries the same factor,
// so it cancels in o / l.
constexpr float kF16Lift = 7.f;

template <int D>
struct __attribute__((aligned(16))) PrefillSmem {
    uint16_t k[2][kTile][D + 8];   // K rows in MFMA row order, 16 B pad per row
    uint16_t v[2][D][kTile];       // V^T: one row of 32 keys per dim, chunks swizzled
    // Exact walk only: bit kk of nf[buf][dim] is set when key t0 + kk of the
    // staged step holds a non-finite V element in that dimension (staged as
    // zero).  Byte c is written by the thread that stages chunk c.
    uint32_t nf[2][D];
};

// V^T row r keeps its four 16-byte chunks in the order c ^ v_swz(r), a
// function of bits 1..3 of r alone
__device__ __forceinline__ int v_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// LDS row of key kk (0..31) of a step: tile a's row n is key 8*(n/4) + n%4,
// tile b's row n (stored at 16 + n) is that key + 4.
__device__ __forceinline__ int k_row(int kk) {
    return ((kk >> 2) & 1) * 16 + 4 * (kk >> 3) + (kk & 3);
}

// A thread's share of one step's K and V: 8 elements per chunk, as bf16
// (16 bytes) or, for an fp8 cache, as E4M3 codes (8 bytes) widened to bf16
// when stored to LDS.
template <int D, int BS, bool FP8>
struct Stage {
    static constexpr int kPasses = D / 64;  // chunks per thread for K (and for V)
    using Word = std::conditional_t<FP8, u32x2, u32x4>;
    Word k[kPasses];
    Word v[kPasses];
};

// Which V^T chunk (dimension, chunk of 8 keys) a thread moves in pass ps.
// With one block per step the four chunks of a dimension go to adjacent
// threads.  With 16-key blocks at D = 128, pass ps covers block ps (keys
// 16ps .. 16ps+15) for every dimension, two threads per dimension, so each
// pass reads from a single block.
template <int D, int BS>
__device__ __forceinline__ void v_chunk(int ps, int tid, int &dim, int &cv) {
    if constexpr (BS == 16 && D == 128) {
        dim = tid >> 1;
        cv = 2 * ps + (tid & 1);
    } else {
        const int idx = ps * 256 + tid;
        dim = idx >> 2;
        cv = idx & 3;
    }
}

// Global -> registers for keys t0 .. t0+31, whose blocks are bidA (keys
// t0 .. t0+15) and bidB (keys t0+16 .. t0+31; the same block unless
// BS == 16).  The step's base addresses are wave-uniform; each thread adds a
// fixed 32-bit offset, so where a pass reads one block the loads take the
// base from scalar registers and no per-lane 64-bit address arithmetic is
// left in the step.  Every call issues the same loads with no branch, so
// the compiler can wait for one stage while the next is in flight: a K row
// or V chunk that lies wholly at or past nkeys is read from the first key
// of its pass's block instead (t0 < nkeys always, and when keys t0+16 .. do
// not exist, bidB is bidA).  Such keys sit past every position of the
// workgroup, so the causal mask drops their scores and stage_store zeroes
// their V elements: they contribute exactly nothing.
// FULL: all 32 keys of the tile exist (the caller checked), so no offset
// needs the clamp.
template <int D, int BS, bool FP8, bool FULL>
__device__ __forceinline__ void stage_load(Stage<D, BS, FP8> &st, const PrefillParams &p,
                                           int kvh, int32_t t0, int32_t nkeys, int32_t bidA,
                                           int32_t bidB, int tid) {
    using E = std::conditional_t<FP8, uint8_t, uint16_t>;  // one stored element
    const E *kc = reinterpret_cast<const E *>(p.k_cache);
    const E *vc = reinterpret_cast<const E *>(p.v_cache);
    const int64_t hkv = p.num_kv_heads;
    const int32_t rowA = t0 % BS, rowB = (t0 + 16) % BS;
    const E *kA = kc + ((bidA * hkv + kvh) * BS + rowA) * D;
    const E *kB = kc + ((bidB * hkv + kvh) * BS + rowB) * D;
    const E *vA = vc + (bidA * hkv + kvh) * (int64_t)D * BS + rowA;
    const E *vB = vc + (bidB * hkv + kvh) * (int64_t)D * BS + rowB;
    const int32_t nvalid = nkeys - t0;  // keys of the tile that exist, >= 1
    // a pass reads a single block: always with BS >= 32; with BS == 16 when
    // D == 128 (K pass ps holds keys 16ps .. 16ps+15, V as v_chunk says)
    constexpr bool kOneBlock = BS >= 32 || D == 128;
#pragma unroll
    for (int ps = 0; ps < Stage<D, BS, FP8>::kPasses; ++ps) {
        const int idx = ps * 256 + tid;
        // K: D/8 chunks of 8 elements per key
        const int kk = idx / (D / 8);
        const int ch = idx % (D / 8);
        int dim, cv;
        v_chunk<D, BS>(ps, tid, dim, cv);
        const E *kp, *vp;
        if constexpr (kOneBlock) {
            // byte offsets from the pass's block base: the thread's own
            // chunk, or the same chunk of the block's first key (K) / the
            // block's first chunk of the dimension (V) when it lies past nkeys
            const int kb0 = BS == 16 ? 16 * ps : 0;  // first key of the pass's block
            const int vb0 = BS == 16 ? 2 * ps : 0;   // its first V chunk
            const uint32_t k_own = (uint32_t)(((kk - kb0) * D + ch * 8) * sizeof(E));
            const uint32_t k_first = (uint32_t)(ch * 8 * sizeof(E));
            const uint32_t v_own = (uint32_t)((dim * BS + 8 * (cv - vb0)) * sizeof(E));
            const uint32_t v_first = (uint32_t)(dim * BS * sizeof(E));
            const char *kbase = reinterpret_cast<const char *>(BS == 16 && ps == 1 ? kB : kA);
            const char *vbase = reinterpret_cast<const char *>(BS == 16 && ps == 1 ? vB : vA);
            kp = reinterpret_cast<const E *>(kbase + (!FULL && kk >= nvalid ? k_first : k_own));
            vp = reinterpret_cast<const E *>(vbase +
                                             (!FULL && 8 * cv >= nvalid ? v_first : v_own));
        } else {
            const int kc_ = kk >= nvalid ? 0 : kk;
            const bool k_in_b = kc_ >= 16;
            kp = (k_in_b ? kB : kA) + (k_in_b ? kc_ - 16 : kc_) * D + ch * 8;
            const int cc = 8 * cv >= nvalid ? 0 : cv;
            const bool v_in_b = cc >= 2;
            vp = (v_in_b ? vB : vA) + dim * BS + 8 * (v_in_b ? cc - 2 : cc);
        }
        if constexpr (FP8) {
            st.k[ps] = ld8(kp);
            st.v[ps] = ld8(vp);
        } else {
            st.k[ps] = ld16(kp);
            st.v[ps] = ld16(vp);
        }
    }
}

// Registers -> LDS.  On the last step (TAIL) the V elements of keys at or
// past nkeys are cleared here rather than right after their load, so the
// loads of a step never wait before the previous step's math; they are
// cleared before any conversion, so no stale value reaches LDS (+0 has the
// same bits in bf16 and fp16).  K is stored as bf16 (an fp8 stage is widened
// exactly).  V is stored as bf16 or, when F16, as fp16: E4M3 codes convert
// exactly, and bf16 elements convert exactly below 2^16 in magnitude; one at
// or past it becomes an fp16 infinity, which the walk's end detects.
// In the exact walk (!F16) a non-finite V element (a bf16 infinity or NaN,
// an E4M3 NaN code) is staged as zero and its key is marked in sm.nf, so
// that the walk can send it only to the columns that see its key.
template <int D, int BS, bool TAIL, bool FP8, bool F16>
__device__ __forceinline__ void stage_store(PrefillSmem<D> &sm, int buf,
                                            const Stage<D, BS, FP8> &st, int tid, int32_t t0,
                                            int32_t nkeys) {
#pragma unroll
    for (int ps = 0; ps < Stage<D, BS, FP8>::kPasses; ++ps) {
        const int idx = ps * 256 + tid;
        const int kk = idx / (D / 8), ch = idx % (D / 8);
        int dim, chv;
        v_chunk<D, BS>(ps, tid, dim, chv);
        u32x4 kw, vw;
        uint32_t nfbits = 0;  // exact walk: element e of the chunk is non-finite
        if constexpr (FP8) {
            kw = e4m3x8_to_bf16x8(st.k[ps]);
            if constexpr (F16) {
                vw = e4m3x8_to_f16x8(st.v[ps]);
            } else {
                // byte b is a NaN code when its low seven bits are all set:
                // adding 1 to those bits then carries into bit 7 (no carry
                // leaves the byte)
                u32x2 c = st.v[ps];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t t = ((c[h] & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
                    c[h] &= ~((t >> 7) * 0xffu);  // NaN codes -> +0
                    nfbits |= (((t >> 7) & 1u) | ((t >> 14) & 2u) | ((t >> 21) & 4u) |
                               ((t >> 28) & 8u)) << (4 * h);
                }
                vw = e4m3x8_to_bf16x8(c);
            }
        } else {
            kw = st.k[ps];
            vw = st.v[ps];
        }
        if constexpr (TAIL) {
            const int32_t t = t0 + 8 * chv;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t keep = (t + 2 * w < nkeys ? 0x0000ffffu : 0u) |
                                      (t + 2 * w + 1 < nkeys ? 0xffff0000u : 0u);
                vw[w] &= keep;
                if constexpr (!F16 && FP8)
                    nfbits &= ~((t + 2 * w < nkeys ? 0u : 1u) << (2 * w) |
                                (t + 2 * w + 1 < nkeys ? 0u : 2u) << (2 * w));
            }
        }
        if constexpr (!F16 && !FP8) {
            // bf16 infinities and NaNs (all exponent bits set) -> +0
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t e = vw[w] & 0x7f807f80u;
                const bool lo_nf = (e & 0xffffu) == 0x7f80u, hi_nf = (e >> 16) == 0x7f80u;
                vw[w] &= (lo_nf ? 0xffff0000u : 0xffffffffu) & (hi_nf ? 0x0000ffffu : 0xffffffffu);
                nfbits |= (lo_nf ? 1u : 0u) << (2 * w) | (hi_nf ? 2u : 0u) << (2 * w);
            }
        }
        if constexpr (!F16)
            reinterpret_cast<uint8_t *>(&sm.nf[buf][dim])[chv] = (uint8_t)nfbits;
        if constexpr (F16 && !FP8) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t lo = vw[w] << 16, hi = vw[w] & 0xffff0000u;
                vw[w] = __builtin_bit_cast(
                    uint32_t, __builtin_convertvector(
                                  f32x2{__uint_as_float(lo), __uint_as_float(hi)}, f16x2));
            }
        }
        *reinterpret_cast<u32x4 *>(&sm.k[buf][k_row(kk)][ch * 8]) = kw;
        *reinterpret_cast<u32x4 *>(&sm.v[buf][dim][8 * (chv ^ v_swz(dim))]) = vw;
    }
}

// Two waves per SIMD (two workgroups per CU): one workgroup's MFMAs run
// while the other waits at its barrier or on LDS.
template <int D, int BS, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8))) void prefill_kernel(
    PrefillParams p) {
    using St = Stage<D, BS, FP8>;
    __shared__ PrefillSmem<D> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const int n = lane & 15, g = lane >> 4;
    const int G = p.num_q_heads / p.num_kv_heads;
    const int ppw = kPairs / G;  // positions per workgroup

    // workgroup -> (kv head fastest, request, chunk slowest): each XCD gets
    // an equal share of kv heads.
    const uint32_t item = blockIdx.x;
    const uint32_t rest = item / (uint32_t)p.num_kv_heads;
    const int kvh = (int)(item - rest * (uint32_t)p.num_kv_heads);
    const int r = (int)(rest % (uint32_t)p.num_reqs);
    const int chunk = (int)(rest / (uint32_t)p.num_reqs);

    const int32_t q0 = p.cu_q_lens[r], q1 = p.cu_q_lens[r + 1];
    if (q0 < 0 || q1 < q0 || q1 > p.total_q_tokens) return;  // no row can be named safely
    const int32_t qlen = q1 - q0;
    const int32_t ctx = p.context_lens[r];
    const int32_t i_begin = chunk * ppw;
    if (i_begin >= qlen) return;

    const bool bad_req = qlen > ctx || qlen > p.max_q_len || ctx > p.max_context_len ||
                         (int64_t)(ctx + BS - 1) / BS > p.table_stride;
    if (bad_req) {
        // NaN for every row this workgroup would own (grid-stride over chunks
        // in case qlen exceeds the bound the grid was sized for).
        const int nchunks = (p.max_q_len + ppw - 1) / ppw;
        const float qnan = __builtin_nanf("");
        for (int32_t rb = i_begin; rb < qlen; rb += nchunks * ppw) {
            const int32_t re = min(qlen, rb + ppw);
            const int64_t elems = (int64_t)(re - rb) * G * D;
            for (int64_t e = tid; e < elems; e += 256) {
                const int32_t row = rb + (int32_t)(e / (G * D));
                const int hg = (int)((e / D) % G), d = (int)(e % D);
                p.out[((int64_t)(q0 + row) * p.num_q_heads + kvh * G + hg) * D + d] = qnan;
            }
        }
        return;
    }

    const int32_t i_end = min(qlen, i_begin + ppw);
    const int32_t base_pos = ctx - qlen;   // absolute position of row 0 of the chunk
    const int32_t nkeys = base_pos + i_end;  // keys 0 .. nkeys-1 are visible to some row

    // This lane's two columns.
    int32_t pos[2];
    int64_t qoff[2];
    // Scores are scaled by |scale| * log2(e) inside the exponent (one fma
    // per weight); a negative scale flips q's sign bits instead, which is
    // exact, so the maximum can be taken on unscaled scores.
    const float sc = fabsf(p.scale_log2);
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
    bf16x8 qb[2][D / 32];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int pair = w * 32 + ct * 16 + n;
        const int hg = pair % G;
        const int32_t ii = i_begin + pair / G;
        const bool valid = pair < ppw * G && ii < i_end;
        pos[ct] = valid ? base_pos + ii : -1;
        qoff[ct] = ((int64_t)(q0 + (valid ? ii : 0)) * p.num_q_heads + kvh * G + hg) * D;
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) + qoff[ct];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            u32x4 v = ld16(qrow + kslot_dim(ks, g)) ^ qsign;
            if (!valid) v = u32x4{0u, 0u, 0u, 0u};
            qb[ct][ks] = as_bf16x8(v);
        }
    }
    // Largest position among this wave's valid columns (-1: none): steps
    // past it hold no key any column of the wave sees.
    int32_t wave_maxpos = -1;
    {
        const int first = w * 32, last = min(w * 32 + 31, ppw * G - 1);
        if (first <= last && i_begin + first / G < i_end)
            wave_maxpos = base_pos + min(i_begin + last / G, i_end - 1);
    }

    const int32_t *table = p.block_tables + (int64_t)r * p.table_stride;
    // Per column tile: running max m, sum l, and two values that change only
    // with m: the rescale threshold m + kRescaleMargin and the exponent base
    // msub (m, or 0 while no key is visible, less the fp16 lift).
    float m[2], l[2], mthr[2], msub[2];
    floatx4 acc[2][D / 16];
    // F16 walk: the sum of each column's weights rides in the matrix core as
    // one more product against a tile whose row 0 is all ones (row 0 of the
    // result, lane (0, n), holds column n's sum of the fp16 weights)
    floatx4 accl[2];
    // Exact walk: bit 4j + i of nfl[ct] marks accumulator acc[ct][j][i] as
    // reached by a non-finite V element of a visible key.
    uint32_t nfl[2] = {0u, 0u};

    // The request's block-table entries live in one VGPR per wave, 64 at a
    // time (lane j holds the entry of logical block win + j); block ids are
    // read with readlane, so no table load stands between a step and its
    // K/V loads.  Entries past the last block of visible keys are not read.
    const int32_t nblk = (nkeys + BS - 1) / BS;
    int32_t win = 0;
    int32_t tbl = 0;
    bool bad = false;
    auto block_id = [&](int32_t j) -> int32_t {
        if (j - win >= 64) {
            win = j;
            tbl = win + lane < nblk ? table[win + lane] : 0;
            // Wait on this path only (vmcnt(0)): the window is then never
            // pending where the paths join, so the steps in between keep
            // their loads in flight across the readlanes below.
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        int32_t b = __builtin_amdgcn_readlane(tbl, j - win);
        if ((uint32_t)b >= (uint32_t)p.num_blocks) {
            bad = true;
            b = 0;
        }
        return b;
    };
    auto stage = [&](St &st, int32_t t0) {
        const int32_t bA = block_id(t0 / BS);
        const int32_t bB = BS == 16 ? block_id(min((t0 + 16) / BS, nblk - 1)) : bA;
        // both branches issue the same loads, so the waits after the join
        // still count one stage
        if (t0 + kTile <= nkeys)
            stage_load<D, BS, FP8, true>(st, p, kvh, t0, nkeys, bA, bB, tid);
        else
            stage_load<D, BS, FP8, false>(st, p, kvh, t0, nkeys, bA, bB, tid);
    };

    const int32_t ntiles = (nkeys + kTile - 1) / kTile;
    const int32_t last_t0 = (ntiles - 1) * kTile;
    // Steps ending at or before the workgroup's first position need no
    // causal mask for any column.  The unmasked run is cut to an even
    // length; a step it leaves over runs with the mask, which is exact.
    const int32_t wg_minpos = base_pos + i_begin;  // first position of the workgroup's rows
    const int32_t nomask = min(ntiles, (wg_minpos + 1) / kTile) & ~1;

    // The whole walk over the keys.  F16: P and V enter the products as
    // fp16; otherwise V stays bf16 and P is split into a bf16 high part and
    // a bf16 remainder.  Returns true when a staged bf16 V element has no
    // exact fp16 value (the F16 result must then be discarded).
    auto run = [&](auto f16_tag) -> bool {
        constexpr bool F16 = decltype(f16_tag)::value;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            m[ct] = kNegInf;
            l[ct] = 0.f;
            accl[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
            mthr[ct] = kNegInf;
            msub[ct] = F16 ? -kF16Lift : 0.f;
            nfl[ct] = 0u;
#pragma unroll
            for (int j = 0; j < D / 16; ++j) acc[ct][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        win = 0;
        tbl = lane < nblk ? table[lane] : 0;

        // Two register stages: while step it computes from LDS, the loads of
        // step it + 2 are in flight and those of step it + 1 (issued one step
        // earlier) are stored to the other LDS buffer at the end of the step,
        // so a load has two steps of math to arrive.
        St stA, stB;
        stage(stA, 0);
        stage(stB, min(kTile, last_t0));  // a tile past the end re-reads the last one, unused
        if (kTile <= nkeys)
            stage_store<D, BS, false, FP8, F16>(sm, 0, stA, tid, 0, nkeys);
        else
            stage_store<D, BS, true, FP8, F16>(sm, 0, stA, tid, 0, nkeys);
        __syncthreads();

        // One 32-key step.  MASK: some column of the workgroup may sit before
        // a key of the step (causal mask needed).
        // cur holds step it + 1's loads, nxt receives step it + 2's.
        auto step = [&](int32_t it, auto mask_tag, St &cur, St &nxt) {
            constexpr bool MASK = decltype(mask_tag)::value;
            const int buf = it & 1;
            const int32_t t0 = it * kTile;
            const bool more = it + 1 < ntiles;
            stage(nxt, min(t0 + 2 * kTile, last_t0));  // past the end: re-read, never stored

            if (wave_maxpos >= t0) {
                u32x4 ka[D / 32], kb[D / 32];
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    ka[ks] = *reinterpret_cast<const u32x4 *>(&sm.k[buf][n][kslot_dim(ks, g)]);
                    kb[ks] =
                        *reinterpret_cast<const u32x4 *>(&sm.k[buf][16 + n][kslot_dim(ks, g)]);
                }
                // Wave priority: the math of a step (Q K^T and the softmax
                // at 2, P V at 1) runs ahead of the co-resident workgroup's
                // staging (its K/V loads, LDS stores and barrier at 0), so a
                // SIMD's two waves keep the matrix core and the vector ALU
                // busy rather than both waiting at barriers.  A/B on the
                // 4 x 512 over 4096 chunk: 190 us with P V alone raised,
                // 179 us with all the math at 1, 178 us as here.
                floatx4 sa[2], sb[2];
                __builtin_amdgcn_s_setprio(2);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    sa[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
                    sb[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < D / 32; ++ks) {
                        sa[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(ka[ks]), qb[ct][ks], sa[ct], 0, 0, 0);
                        sb[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(kb[ks]), qb[ct][ks], sb[ct], 0, 0, 0);
                    }
                }
                u32x4 vv[D / 16];
#pragma unroll
                for (int j = 0; j < D / 16; ++j)
                    vv[j] = *reinterpret_cast<const u32x4 *>(&sm.v[buf][16 * j + n][8 * (g ^ v_swz(n))]);
                u32x4 ph[2], pl[2];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    float sr[8];  // unscaled scores of keys t0 + 8g + i
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sr[i] = sa[ct][i];
                        sr[4 + i] = sb[ct][i];
                    }
                    bool vis[8];
                    float mr = kNegInf;  // this lane's largest visible score
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        vis[i] = !MASK || t0 + 8 * g + i <= pos[ct];
                        mr = fmaxf(mr, vis[i] ? sr[i] : kNegInf);
                    }
                    // Lazy rescaling: the exponent base m[ct] moves only when
                    // a weight of the step would reach 2^kRescaleMargin, so
                    // the accumulators are rescaled on few steps.  The test
                    // needs no cross-lane max: if no lane's own max passes
                    // the bound, every weight of the column stays below it.
                    // When some lane's does (a wave-uniform branch), the
                    // exact column max becomes the new base of every column.
                    if (__any(mr * sc > mthr[ct])) {
                        const float cm = rows4_max(mr);
                        const float mx = cm == kNegInf ? kNegInf : cm * sc;
                        const float m_new = fmaxf(m[ct], mx);
                        const float f = m_new == kNegInf ? 1.f : fast_exp2(m[ct] - m_new);
                        if constexpr (F16)
                            accl[ct] *= f;
                        else
                            l[ct] *= f;
#pragma unroll
                        for (int j = 0; j < D / 16; ++j) acc[ct][j] *= f;
                        m[ct] = m_new;
                        mthr[ct] = m_new + kRescaleMargin;
                        msub[ct] = (m_new == kNegInf ? 0.f : m_new) - (F16 ? kF16Lift : 0.f);
                    }
                    // A column with no visible key yet keeps m = -inf; its
                    // weights are all exp2(-inf) = 0, so any finite base
                    // serves.  F16 lifts every weight by 2^kF16Lift.
                    float pv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float arg = fmaf(sr[i], sc, -msub[ct]);
                        pv[i] = fast_exp2(MASK && !vis[i] ? kNegInf : arg);
                    }
                    if constexpr (F16) {
                        // P rounded to fp16 (nearest even)
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            ph[ct][k] = __builtin_bit_cast(
                                uint32_t,
                                __builtin_convertvector(f32x2{pv[2 * k], pv[2 * k + 1]}, f16x2));
                    } else {
                        // P = hi + lo: hi keeps the top 16 bits of each fp32
                        // weight (a bf16 value), lo = P - hi is exact in fp32
                        // and rounded to bf16, so P enters the bf16 products
                        // with ~16 bits.
                        uint32_t hb[8];
                        float lo[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            hb[i] = __float_as_uint(pv[i]);
                            lo[i] = pv[i] - __uint_as_float(hb[i] & 0xffff0000u);
                        }
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            ph[ct][k] = __builtin_amdgcn_perm(hb[2 * k + 1], hb[2 * k], 0x07060302u);
                            pl[ct][k] = __builtin_bit_cast(
                                uint32_t,
                                __builtin_convertvector(f32x2{lo[2 * k], lo[2 * k + 1]}, bf16x2));
                        }
                        l[ct] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) +
                                 ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                    }
                }
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int j = 0; j < D / 16; ++j) {
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        if constexpr (F16) {
                            acc[ct][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                as_f16x8(vv[j]), as_f16x8(ph[ct]), acc[ct][j], 0, 0, 0);
                        } else {
                            acc[ct][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(vv[j]), as_bf16x8(ph[ct]), acc[ct][j], 0, 0, 0);
                            acc[ct][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(vv[j]), as_bf16x8(pl[ct]), acc[ct][j], 0, 0, 0);
                        }
                    }
                }
                if constexpr (!F16) {
                    // Non-finite V elements were staged as zeros.  Accumulator
                    // (dim, column) is marked when one of them sits at a key the
                    // column sees (keys t0 .. pos); marked outputs become NaN,
                    // and no other column is touched by them.
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        const int32_t rel = pos[ct] - t0;
                        const uint32_t vm = rel < 0 ? 0u : rel >= 31 ? ~0u : (2u << rel) - 1u;
#pragma unroll
                        for (int j = 0; j < D / 16; ++j) {
                            const u32x4 nm =
                                *reinterpret_cast<const u32x4 *>(&sm.nf[buf][16 * j + 4 * g]);
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                nfl[ct] |= (nm[i] & vm) != 0u ? 1u << (4 * j + i) : 0u;
                        }
                    }
                }
                if constexpr (F16) {
                    const uint32_t one2 = n == 0 ? 0x3c003c00u : 0u;  // fp16 1.0 pairs in row 0
                    const u32x4 ones = {one2, one2, one2, one2};
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
                        accl[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            as_f16x8(ones), as_f16x8(ph[ct]), accl[ct], 0, 0, 0);
                }
                __builtin_amdgcn_s_setprio(0);
            }
            if (more) {
                if (t0 + 2 * kTile <= nkeys)
                    stage_store<D, BS, false, FP8, F16>(sm, buf ^ 1, cur, tid, t0 + kTile, nkeys);
                else
                    stage_store<D, BS, true, FP8, F16>(sm, buf ^ 1, cur, tid, t0 + kTile, nkeys);
            }
            __syncthreads();
        };
        // Even steps find step it + 1 in stB, odd steps in stA.  The loop
        // runs steps in pairs so each body names its stages at compile time:
        // the two are never copied into each other or selected at run time,
        // and each wait covers one stage's loads.
        int32_t it = 0;
        for (; it < nomask; it += 2) {
            step(it, std::false_type{}, stB, stA);
            step(it + 1, std::false_type{}, stA, stB);
        }
        for (; it < ntiles; it += 2) {
            step(it, std::true_type{}, stB, stA);
            if (it + 1 < ntiles) step(it + 1, std::true_type{}, stA, stB);
        }
        if constexpr (F16) {
            // A staged bf16 V element of magnitude 2^16 or more (the first
            // one past fp16's 65504) became an fp16 infinity; an infinite or
            // NaN bf16 element or an E4M3 NaN code is staged as it is.  Every
            // staged key is in a step that some wave of the workgroup
            // computes, and any fp16 weight, zero included, times an infinity
            // or a NaN is an infinity or a NaN, so such an element leaves a
            // non-finite value in that wave's accumulators whether or not
            // the wave's columns see its key (a masked key's zero weight
            // gives 0 * inf = NaN); rescaling and later sums keep it
            // non-finite.  With every element finite and below 2^16 the sums
            // stay far inside fp32's range (weights below 2^15 here), so a
            // non-finite sum of a lane's accumulators means the fp16 walk's
            // result cannot be kept.
            float s = 0.f;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int j = 0; j < D / 16; ++j)
                    s += (acc[ct][j][0] + acc[ct][j][1]) + (acc[ct][j][2] + acc[ct][j][3]);
            return __syncthreads_or(__builtin_isfinite(s) ? 0 : 1) != 0;
        } else {
            return false;
        }
    };
    // fp16 walk first.  A workgroup that staged a V element the fp16 walk
    // cannot carry exactly (beyond fp16's range, or not finite) walks again
    // with the exact products and non-finite elements kept to the columns
    // that see them.
    bool f16_walk = true;
    if (run(std::true_type{})) {
        run(std::false_type{});
        f16_walk = false;
    }

    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const float lt = f16_walk ? __shfl(accl[ct][0], n, 64) : rows4_sum(l[ct]);
        if (pos[ct] < 0) continue;
        const float inv = (FP8 ? p.v_scale : 1.f) / lt;  // an fp8 V scale enters here
        float *orow = p.out + qoff[ct];
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            floatx4 o = acc[ct][j] * inv;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((nfl[ct] >> (4 * j + i)) & 1u) o[i] = qnan;
            if (any_bad) o = floatx4{qnan, qnan, qnan, qnan};
            *reinterpret_cast<floatx4 *>(orow + 16 * j + 4 * g) = o;
        }
    }
}

template <int D, int BS>
int launch_one(const PrefillParams &p, hipStream_t s) {
    const int G = p.num_q_heads / p.num_kv_heads;
    const int ppw = kPairs / G;
    const int64_t nchunks = (p.max_q_len + ppw - 1) / ppw;
    const int64_t wgs = nchunks * p.num_reqs * p.num_kv_heads;
    if (wgs > (1LL << 24) - 1) return -1;
    if (p.kv_fp8)
        hipLaunchKernelGGL((prefill_kernel<D, BS, true>), dim3((unsigned)wgs), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_kernel<D, BS, false>), dim3((unsigned)wgs), dim3(256), 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_prefill(const PrefillParams &p, void *stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#define PA_CASE(Dv, BSv) \
    if (p.head_dim == Dv && p.block_size == BSv) return launch_one<Dv, BSv>(p, s);
    PA_CASE(128, 16) PA_CASE(128, 32) PA_CASE(128, 64) PA_CASE(128, 128)
    PA_CASE(64, 16) PA_CASE(64, 32) PA_CASE(64, 64) PA_CASE(64, 128)
#undef PA_CASE
    return -1;
}

}  // namespace pa
