// Decode attention over a paged KV cache, one query token per sequence.
//
// "vLLM and PagedAttention" slide 9: attention is evaluated one block at a
// time, with keys and values read from physically scattered blocks located
// through the block table (slide 10). The result is ordinary single-query scaled
// dot-product attention over the sequence's gathered context.
//
// Kernel design (gfx950, wave64), one workgroup of W waves per
// (sequence, query head[, partition]):
//  * the work unit is a tile: TR consecutive rows (tokens) of one
//    (block, kv head), TR * head_dim contiguous elements; the tiles of the
//    workgroup's token range are dealt round-robin to its waves;
//  * a lane reads 16 bytes per load, consecutive lanes on consecutive 16 bytes,
//    so one load instruction covers RPI whole rows (1 KiB for 16-bit d=128);
//    K and V loads are non-temporal (each byte is read once);
//  * each wave keeps 64 of its block-table entries in one register (lane i
//    holds its i-th next entry) and moves an entry to a scalar register with
//    readlane, so a tile's base address is scalar and no LDS or barrier sits
//    in the loop;
//  * loads are double-buffered in registers: the next stage's K/V loads are in
//    flight while the current stage is consumed;
//  * a row's dot product is split over LPR lanes (dot2 instructions for 16-bit
//    types) and summed with DPP row operations; softmax is online per lane
//    (running max m, sum l, rescaled accumulator) in base 2 with log2(e)
//    folded into the scale; lanes, then waves, are merged in a fixed order at
//    the end: no atomics, so results are bit-reproducible and do not depend on
//    where blocks live;
//  * rows past the context end are never loaded and are excluded by select,
//    never multiplied by a zero weight (0 * NaN = NaN);
//  * split mode: each partition writes (m, l, unnormalised accumulator) to an
//    fp32 workspace and a second kernel merges them:
//    M = max_p m_p, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// The contiguous-cache variant is the same template; only a tile's address
// differs.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "attention.h"

namespace pkv {
namespace {

constexpr int kWaves = 12;  // per-item schedule: one workgroup of three waves per SIMD on each CU
constexpr int kThreads = kWaves * 64;
constexpr int kWavesNarrow = 4;       // per-item schedule, short fixed partitions: three workgroups per CU
constexpr int kSplitTilesNarrow = 32;  // partitions of at most this many tiles take the narrow workgroup

template <class E, int D, int B>
struct Shape {
    static constexpr int VEC = E::VEC;                  // elements per 16-byte load
    static constexpr int LPR = D / VEC;                 // lanes per row
    static constexpr int RPI = 64 / LPR;                // rows per load instruction
    static constexpr int TR = B < RPI * 4 ? B : RPI * 4;  // tile rows: at most 4 loads per lane per tile
    static constexpr int SPB = B / TR;                  // tiles per block
    static constexpr int NL = TR / RPI;                 // loads per lane per tile (K or V)
    static constexpr int U = 4 / NL;                    // tiles per stage: 4 K and 4 V loads per lane
    static constexpr int TILE_ELEMS = TR * D;
    static_assert(LPR >= 8 && LPR <= 64 && 64 % LPR == 0, "head_dim does not map onto a wave");
    static_assert(TR % RPI == 0 && B % TR == 0, "block_size must be a multiple of rows per load");
    static_assert(64 % U == 0, "a stage must not straddle a table chunk");
};

template <int W, int D>
struct MhaLds {
    float m[W], l[W];
    float acc[W][D];
};

// Tokens [t0, t1) of sequence s for query head h (t0 a multiple of the tile rows, t0 < t1 <= the
// length): the workgroup's merged result goes to sink. Uniform over the workgroup; ends with a
// barrier, so the caller may run it again on the same LDS. In a decode step with the cache write,
// the one caller per (sequence, kv head) that passes write_new stores the sequence's new rows.
template <class E, int D, int B, bool PAGED, int W, int POL>
__device__ inline void mha_range(const AttnParams &p, int s, int h, int t0, int t1, const Sink &sink,
                                 MhaLds<W, D> &lds, bool write_new) {
    using SH = Shape<E, D, B>;
    constexpr int VEC = SH::VEC, LPR = SH::LPR, RPI = SH::RPI, TR = SH::TR, SPB = SH::SPB, NL = SH::NL,
                  U = SH::U;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers, scalar branches
    const int kvh = h / p.group;
    const int64_t row_q = static_cast<int64_t>(s) * p.num_q_heads + h;
    const int r0 = lane / LPR, c = lane % LPR;

    // Tiles of this workgroup: jt0 .. jt0+n-1 (tile jt covers tokens jt*TR .. jt*TR+TR-1);
    // this wave takes tiles jt0 + wave + k*W, k = 0 .. nk-1, in stages of U tiles.
    const int jt0 = t0 / TR;

    // Block-table chunk: lane i holds the physical block of this wave's tile kc0 + i. A lane whose
    // tile lies past the range's last block (t1 <= the length) reads no entry and holds 0, which
    // no tile uses.
    const int32_t *trow = PAGED ? p.tables + static_cast<int64_t>(s) * p.max_blocks : nullptr;
    const int jlast = (t1 - 1) / B;  // the range's last block (< max_blocks: t1 <= ctx_cap)
    int tb = 0;
    auto fetch_table = [&](int base) -> int {
        const int j = (jt0 + wave + (base + lane) * W) / SPB;
        return j <= jlast ? trow[j] : 0;
    };
    if constexpr (PAGED) tb = fetch_table(0);
    // tokens below clen are loaded through the caches (uniform: a scalar compare per tile)
    const int clen = POL == kLoadSplit ? __builtin_amdgcn_readfirstlane(p.cached_lens[s]) : 0;
    const u32x4 qv = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.q) + (row_q * D + c * VEC) * E::ELT);
    // decode step with the cache write: the sequence's last row (its new token), when this launch
    // writes it, comes from the new key and value rows (chunk c in every lane), not from the cache
    // (the loads go out without waiting for the position, which is first needed at the last stage)
    const int last = new_row_position(p, s);
    u32x4 knew = {0u, 0u, 0u, 0u}, vnew = {0u, 0u, 0u, 0u};
    if (p.new_k) {
        const int64_t nrow = (static_cast<int64_t>(s) * p.num_kv_heads + kvh) * D + c * VEC;
        knew = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.new_k) + nrow * E::ELT);
        vnew = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.new_v) + nrow * E::ELT);
    }

    const char *kc = static_cast<const char *>(p.k);
    const char *vc = static_cast<const char *>(p.v);
    const int n = (t1 + TR - 1) / TR - jt0;
    const int nk = n > wave ? (n - wave + W - 1) / W : 0;  // tiles of this wave

    // Byte offset of this wave's tile k, whose table entry is lane k - kc0 of the current
    // chunk; ok = false for a table entry outside the pool.
    auto tile_offset = [&](int k, int kc0, bool &ok) -> int64_t {
        const int jt = jt0 + wave + k * W;
        if constexpr (PAGED) {
            const int pb = __builtin_amdgcn_readlane(tb, k - kc0);
            ok = static_cast<uint32_t>(pb) < p.num_blocks;  // 32-bit, so it stays a scalar compare
            const int64_t blk = ok ? pb : 0;
            return ((blk * p.num_kv_heads + kvh) * B + (jt % SPB) * TR) * D * E::ELT;
        } else {
            ok = true;
            return ((static_cast<int64_t>(s) * p.num_kv_heads + kvh) * p.lmax + static_cast<int64_t>(jt) * TR) * D *
                   E::ELT;
        }
    };

    struct Stage {
        u32x4 k[U][NL], v[U][NL];
        int tok0[U];
        bool ok[U];  // table entry inside the pool
        bool in[U];  // tile belongs to this wave (false: a stand-in, masked out)
    };

    // Every load is unconditional, so the compiler's wait counts stay exact. With clamp set, a
    // tile past the wave's last is replaced by its last tile and a row at or past t1 by the
    // row before t1: both in bounds and written; consume() masks them out.
    auto issue = [&](Stage &S, int kc0, int st, bool clamp) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int k = kc0 + st * U + u;
            S.in[u] = k < nk;
            if (clamp) k = min(k, nk - 1);
            const int64_t tile = tile_offset(k, kc0, S.ok[u]);
            const char *kt = kc + tile, *vt = vc + tile;  // uniform: a scalar base for the loads
            S.tok0[u] = (jt0 + wave + k * W) * TR;
            const int lim = t1 - 1 - S.tok0[u];  // last row inside the context
            unsigned off[NL];
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const unsigned row = clamp ? min(l * RPI + r0, lim) : l * RPI + r0;
                off[l] = row * (D * E::ELT) + c * (VEC * E::ELT);
            }
            if (POL == kLoadCached || (POL == kLoadSplit && S.tok0[u] < clen)) {
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    S.k[u][l] = kv_load<false>(kt + off[l]);
                    S.v[u][l] = kv_load<false>(vt + off[l]);
                }
            } else {
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    S.k[u][l] = kv_load<true>(kt + off[l]);
                    S.v[u][l] = kv_load<true>(vt + off[l]);
                }
            }
        }
    };

    float m = -INFINITY, lsum = 0.f;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

    auto consume = [&](Stage &S, bool tail) {
        if (tail && last >= 0) {  // the last row lies in a wave's last stage
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (S.tok0[u] > last || last >= S.tok0[u] + TR) continue;  // uniform
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    // the row this lane loaded: rows at or past t1 were clamped to row t1 - 1, and
                    // their zero weights would not cancel a stale value there (0 * NaN = NaN)
                    const bool mine = S.tok0[u] + min(l * RPI + r0, t1 - 1 - S.tok0[u]) == last;
                    S.k[u][l] = mine ? knew : S.k[u][l];
                    S.v[u][l] = mine ? vnew : S.v[u][l];
                }
            }
        }
        float sc[U][NL];
        float mloc = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const float d = group_sum<LPR>(E::dot(qv, S.k[u][l], 0.f)) * p.scale_log2;
                const bool valid = S.ok[u] && (!tail || (S.in[u] && S.tok0[u] + l * RPI + r0 < t1));
                sc[u][l] = valid ? d : -INFINITY;
                mloc = fmaxf(mloc, sc[u][l]);
            }
        }
        const float m_new = fmaxf(m, mloc);
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // a lane with no valid row yet
        const float alpha = fast_exp2(m - m_ref);
        lsum *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // uniform: a rejected table entry's tile and a stand-in tile are never accumulated
            if (!S.ok[u] || (tail && !S.in[u])) continue;
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const float pr = fast_exp2(sc[u][l] - m_ref);
                lsum += pr;
                E::axpy(pr, S.v[u][l], acc);
            }
        }
        m = m_new;
    };

    // The wave's tiles in chunks of 64 (one table register each); within a chunk, stages of U
    // tiles are double-buffered. All stages but a wave's last are full (every tile exists and
    // every row is inside the context), so the steady-state loop needs no clamping or masks.
    for (int kc0 = 0; kc0 < nk; kc0 += 64) {
        if constexpr (PAGED) {
            if (kc0 > 0) tb = fetch_table(kc0);
        }
        const int nst = (min(64, nk - kc0) + U - 1) / U;
        const bool last_chunk = kc0 + 64 >= nk;
        Stage A, Bs;
        int st = 0;
        issue(A, kc0, 0, last_chunk && nst < 2);
        while (st + 4 <= nst) {
            issue(Bs, kc0, st + 1, false);
            consume(A, false);
            // keep the next stage's loads behind this consume: two stages in registers, not three
            __builtin_amdgcn_sched_barrier(0);
            issue(A, kc0, st + 2, false);
            consume(Bs, false);
            __builtin_amdgcn_sched_barrier(0);
            st += 2;
        }
        // 1 to 3 stages remain (A holds the first); straight-line code per case keeps every
        // issue unconditional
        switch (nst - st) {
        case 1:
            consume(A, true);
            break;
        case 2:
            issue(Bs, kc0, st + 1, true);
            consume(A, true);
            consume(Bs, true);
            break;
        default:
            issue(Bs, kc0, st + 1, true);
            consume(A, true);
            issue(A, kc0, st + 2, true);
            consume(Bs, true);
            consume(A, true);
            break;
        }
    }

    // Merge the lane groups that hold the same columns (different rows), in a fixed order.
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
        const float mo = __shfl_xor(m, o), lo = __shfl_xor(lsum, o);
        const float M = fmaxf(m, mo);
        const float Mr = M == -INFINITY ? 0.f : M;
        const float f1 = fast_exp2(m - Mr), f2 = fast_exp2(mo - Mr);
        lsum = lsum * f1 + lo * f2;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = acc[e] * f1 + __shfl_xor(acc[e], o) * f2;
        m = M;
    }
    if (lane < LPR) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) lds.acc[wave][c * VEC + e] = acc[e];
    }
    if (lane == 0) {
        lds.m[wave] = m;
        lds.l[wave] = lsum;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < D; i += W * 64) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, lds.m[w]);
        const float Mr = M == -INFINITY ? 0.f : M;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = fast_exp2(lds.m[w] - Mr);
            L = fmaf(lds.l[w], f, L);
            O = fmaf(lds.acc[w][i], f, O);
        }
        if (sink.acc) {
            sink.acc[i] = O;
            if (i == 0) {
                sink.m[0] = M;
                sink.l[0] = L;
            }
        } else {
            E::store(p.out, row_q * D + i, L > 0.f ? O / L : 0.f);
        }
    }
    __syncthreads();
    // after the barrier, which would otherwise wait for these stores to complete
    if (write_new && last >= 0 && wave == 0 && lane < LPR)  // lanes 0 .. LPR-1 hold the whole row
        store_new_row<B, D * E::ELT>(p, s, kvh, c, knew, vnew);
}

// Per-item schedule: grid = (num_q_heads, num_seqs, parts), block = 64 * W; one workgroup per
// (sequence, query head[, partition]).
template <class E, int D, int B, bool PAGED, int W, int POL>
__global__ __launch_bounds__(W * 64) void attn_decode_kernel(const AttnParams p) {
    __shared__ MhaLds<W, D> lds;
    const int h = blockIdx.x, s = blockIdx.y, part = blockIdx.z;
    const int64_t row_q = static_cast<int64_t>(s) * p.num_q_heads + h;
    const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
    const int t0 = p.partition_size > 0 ? part * p.partition_size : 0;
    const int t1 = p.partition_size > 0 ? min(ctx, t0 + p.partition_size) : ctx;
    if (t0 >= t1) {  // uniform over the workgroup
        if (p.partition_size == 0)
            for (int i = threadIdx.x; i < D; i += W * 64) E::store(p.out, row_q * D + i, 0.f);
        return;
    }
    Sink sink{nullptr, nullptr, nullptr, 0, 0};
    if (p.partition_size > 0) {
        const int64_t wr = row_q * p.num_parts + part;
        sink = Sink{p.ws + wr * D, p.ws + p.ws_rows * D + wr, p.ws + p.ws_rows * (D + 1) + wr, 0, 0};
    }
    // one workgroup per (sequence, kv head) writes the new rows of a decode step
    mha_range<E, D, B, PAGED, W, POL>(p, s, h, t0, t1, sink, lds, t0 == 0 && h % p.group == 0);
}

// Balanced schedule: grid = balanced_wgs workgroups, each an equal share of the batch's tiles
// (work rows = (sequence, query head)); cut rows are merged by attn_reduce_balanced_kernel.
template <class E, int D, int B, bool PAGED, int W, int POL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_decode_balanced_kernel(
    const AttnParams p) {
    __shared__ MhaLds<W, D> lds;
    __shared__ uint32_t C[kBalancedMaxSeqs + 1];
    __shared__ uint32_t part[W * 64];
    balanced_prefix<W * 64>(p, C, part, balanced_prefix_out(p));
    balanced_zero_empty<E, D, W * 64>(p, C);
    balanced_walk<D, false>(p, C, [&](int s, int h, int ta, int tb, const Sink &sink) {
        constexpr int TR = Shape<E, D, B>::TR;
        const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
        // the share holding a row's first tile writes the new rows of a decode step
        mha_range<E, D, B, PAGED, W, POL>(p, s, h, ta * TR, min(tb * TR, ctx), sink, lds, ta == 0 && h % p.group == 0);
    });
}

// Merge of the partitions of one (sequence, head): grid = (num_q_heads, num_seqs), block = D.
template <class E, int D>
__global__ __launch_bounds__(D) void attn_reduce_kernel(const AttnParams p) {
    const int h = blockIdx.x, s = blockIdx.y, i = threadIdx.x;
    const int64_t row_q = static_cast<int64_t>(s) * p.num_q_heads + h;
    const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
    const int np = (ctx + p.partition_size - 1) / p.partition_size;
    const float *wacc = p.ws + row_q * p.num_parts * D;
    const float *wm = p.ws + p.ws_rows * D + row_q * p.num_parts;
    const float *wl = p.ws + p.ws_rows * (D + 1) + row_q * p.num_parts;
    float M = -INFINITY;
    for (int j = 0; j < np; ++j) M = fmaxf(M, wm[j]);
    const float Mr = M == -INFINITY ? 0.f : M;
    float L = 0.f, O = 0.f;
    for (int j = 0; j < np; ++j) {
        const float f = fast_exp2(wm[j] - Mr);
        L = fmaf(wl[j], f, L);
        O = fmaf(wacc[static_cast<int64_t>(j) * D + i], f, O);
    }
    E::store(p.out, row_q * D + i, L > 0.f ? O / L : 0.f);
}

// The balanced schedule's merge: grid = balanced_wgs, block = 256. Share v merges the cut row
// whose last tile it holds (if any), from the partial results of the shares that hold parts of
// it, in share order. Rows held whole by one share were written by it; rows of sequences with
// no tokens were zeroed by the attention kernel.
template <class E, int D>
__global__ __launch_bounds__(256) void attn_reduce_balanced_kernel(const AttnParams p) {
    const int64_t v = blockIdx.x;
    const int32_t *rec = balanced_records(p) + 2 * v;
    const int s = rec[0], row = rec[1];
    if (s < 0) return;
    const uint32_t *C = balanced_prefix_out(p);  // written by the attention kernel's workgroup 0
    const int64_t R = p.rows_per_seq, nwg = p.balanced_wgs, Ctot = C[p.num_seqs], T = R * Ctot;
    const int64_t n = C[s + 1] - C[s];
    const int H = p.heads_per_row;
    const int64_t row_q0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(row) * H;
    const int64_t row0 = p.head_major ? row * Ctot + C[s] : R * C[s] + row * n;
    const int64_t g0 = balanced_owner(row0, T, nwg), g1 = v;
    const int64_t slot_floats = static_cast<int64_t>(H) * (D + 2);
    // the first share's part of this row is its first row only if the share starts on the row
    const int64_t first_slot = balanced_begin(g0, T, nwg) < row0 ? 2 * g0 + 1 : 2 * g0;
    // shares with an empty range (more shares than tiles) hold nothing and are skipped
    auto empty = [&](int64_t g) { return balanced_begin(g + 1, T, nwg) == balanced_begin(g, T, nwg); };
    for (int i = threadIdx.x; i < H * D; i += 256) {
        const int j = i / D, d = i % D;
        // one pass over the shares with a running max (the shares' loads are independent)
        float M = -INFINITY, L = 0.f, O = 0.f;
        for (int64_t g = g0; g <= g1; ++g) {
            if (empty(g)) continue;
            const float *slot = p.ws + (g == g0 ? first_slot : 2 * g) * slot_floats;
            const float mg = slot[H * D + j], lg = slot[H * (D + 1) + j], og = slot[j * D + d];
            const float Mn = fmaxf(M, mg);
            const float Mr = Mn == -INFINITY ? 0.f : Mn;
            const float a = fast_exp2(M - Mr), f = fast_exp2(mg - Mr);
            L = fmaf(lg, f, L * a);
            O = fmaf(og, f, O * a);
            M = Mn;
        }
        E::store(p.out, (row_q0 + j) * D + d, L > 0.f ? O / L : 0.f);
    }
}

constexpr int kBalancedWaves = 4;

template <class E, int D, int B, bool PAGED, int POL>
int launch(const AttnParams &p, int32_t num_seqs, int32_t grid_parts, hipStream_t stream) {
    if (p.partition_size == PKV_PARTITION_BALANCED) {
        AttnParams q = p;
        q.tile_rows = Shape<E, D, B>::TR;
        q.rows_per_seq = p.num_q_heads;
        q.heads_per_row = 1;
        q.head_major = 0;
        int rc = balanced_check(q);
        if (rc) return rc;
        hipLaunchKernelGGL((attn_decode_balanced_kernel<E, D, B, PAGED, kBalancedWaves, POL>), dim3(q.balanced_wgs),
                           dim3(kBalancedWaves * 64), 0, stream, q);
        rc = hip_status(hipGetLastError(), "attention launch");
        return rc ? rc : launch_reduce_balanced(q, E::CODE, D, stream);
    }
    if (grid_parts > 65535)
        return fail(PKV_EINVAL, "attention: %d partitions per sequence exceed the grid (65535)", grid_parts);
    // Grid (heads, sequences, partitions): workgroups are dealt to the XCDs round-robin in this
    // order, so each XCD serves every eighth head across all sequences and partitions, an even
    // share. (Partitions fastest would give each XCD a fixed partition index, and the later
    // partitions exist only for the longer sequences.) A fixed partition of at most 32 tiles goes
    // to 4 waves, so each still walks up to 8 tiles through its register pipeline; longer ranges
    // (one pass, larger partitions) to 12.
    constexpr int TR = Shape<E, D, B>::TR;
    const dim3 grid(p.num_q_heads, num_seqs, grid_parts);
    if (p.partition_size > 0 && p.partition_size <= kSplitTilesNarrow * TR)
        hipLaunchKernelGGL((attn_decode_kernel<E, D, B, PAGED, kWavesNarrow, POL>), grid, dim3(kWavesNarrow * 64), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((attn_decode_kernel<E, D, B, PAGED, kWaves, POL>), grid, dim3(kThreads), 0, stream, p);
    int rc = hip_status(hipGetLastError(), "attention launch");
    if (rc || p.partition_size <= 0) return rc;
    return launch_reduce(p, E::CODE, D, num_seqs, stream);
}

template <class E, int D, bool PAGED>
int dispatch_block(const AttnParams &p, int32_t block_size, int pol, int32_t num_seqs, int32_t grid_parts,
                   hipStream_t stream) {
    if constexpr (!PAGED) {
        return launch<E, D, 16, false, kLoadStream>(p, num_seqs, grid_parts, stream);  // 16-row tiles
    } else {
#define PKV_B(B)                                                                                      \
    return pol == kLoadCached  ? launch<E, D, B, true, kLoadCached>(p, num_seqs, grid_parts, stream) \
           : pol == kLoadSplit ? launch<E, D, B, true, kLoadSplit>(p, num_seqs, grid_parts, stream)  \
                               : launch<E, D, B, true, kLoadStream>(p, num_seqs, grid_parts, stream)
        switch (block_size) {
        case 8: PKV_B(8);
        case 16: PKV_B(16);
        case 32: PKV_B(32);
        default: return fail(PKV_EUNSUPPORTED, "block_size %d not built (8, 16, 32)", block_size);
        }
#undef PKV_B
    }
}

// One query head per workgroup (any G), then the merge pass of the split modes.
template <bool PAGED>
int dispatch_per_head(const AttnParams &p, int32_t dtype, int32_t head_dim, int32_t block_size, int pol,
                      int32_t num_seqs, int32_t grid_parts, hipStream_t stream) {
    int rc;
#define PKV_HD(E)                                                                                 \
    switch (head_dim) {                                                                           \
    case 64: rc = dispatch_block<E, 64, PAGED>(p, block_size, pol, num_seqs, grid_parts, stream); break; \
    case 128: rc = dispatch_block<E, 128, PAGED>(p, block_size, pol, num_seqs, grid_parts, stream); break; \
    default: return fail(PKV_EUNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);          \
    }
    switch (dtype) {
    case PKV_F32: PKV_HD(F32) break;
    case PKV_F16: PKV_HD(F16) break;
    case PKV_BF16: PKV_HD(BF16) break;
    default: return fail(PKV_EINVAL, "bad dtype %d", dtype);
    }
#undef PKV_HD
    return rc;
}

template <bool PAGED>
int dispatch(const AttnParams &p, int32_t dtype, int32_t head_dim, int32_t block_size, int32_t num_seqs,
             int32_t grid_parts, uint32_t flags, hipStream_t stream) {
    const int pol = !PAGED                          ? kLoadStream
                    : (flags & PKV_FLAG_CACHED_KV) ? kLoadCached
                    : p.cached_lens                ? kLoadSplit
                                                   : kLoadStream;
    if (p.group > 1 && !(flags & PKV_FLAG_SCALAR_GQA) && gqa_mfma_supported(dtype, head_dim, block_size, p.group))
        return launch_gqa_mfma(p, dtype, block_size, PAGED, pol, num_seqs, grid_parts, stream);
    return dispatch_per_head<PAGED>(p, dtype, head_dim, block_size, pol, num_seqs, grid_parts, stream);
}

// Checks shared by the paged and contiguous entry points.
int check_common(const char *fn, const void *out, const void *q, const void *k, const void *v,
                 const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, float scale, int32_t partition_size, void *workspace,
                 size_t workspace_bytes, int32_t dtype) {
    if (!valid_dtype(dtype)) return fail(PKV_EINVAL, "%s: bad dtype %d", fn, dtype);
    if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "%s: num_seqs %d outside [0, 65535]", fn, num_seqs);
    if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads || num_q_heads > 65535)
        return fail(PKV_EINVAL, "%s: num_q_heads %d must be a positive multiple of num_kv_heads %d", fn,
                    num_q_heads, num_kv_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_EUNSUPPORTED, "%s: head_dim %d not built (64, 128)", fn, head_dim);
    if (max_context_len < 0) return fail(PKV_EINVAL, "%s: max_context_len < 0", fn);
    if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale is not finite", fn);
    if (partition_size < 0 && partition_size != PKV_PARTITION_BALANCED)
        return fail(PKV_EINVAL, "%s: partition_size %d (0, > 0, or PKV_PARTITION_BALANCED)", fn, partition_size);
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k || !v || !context_lens) return fail(PKV_EINVAL, "%s: NULL pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(PKV_EINVAL, "%s: out, q, k, v must be 16-byte aligned", fn);
    if (partition_size != 0) {
        // (the balanced mode's exact need depends on the kernel chosen; it is checked again at launch)
        const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size);
        if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
            return fail(PKV_EINVAL, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn, need,
                        workspace ? workspace_bytes : 0);
    }
    return PKV_OK;
}

AttnParams make_params(void *out, const void *q, const void *k, const void *v, const int32_t *context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, float scale,
                       int32_t partition_size, int32_t max_context_len, int32_t ctx_cap, void *workspace,
                       size_t workspace_bytes, int32_t head_dim) {
    AttnParams p{};
    p.out = out;
    p.q = q;
    p.k = k;
    p.v = v;
    p.ctx_lens = context_lens;
    p.ctx_cap = ctx_cap;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.partition_size = ctx_cap > 0 ? partition_size : 0;
    p.num_parts = partition_size > 0 ? static_cast<int32_t>(ceil_div(max_context_len, partition_size)) : 0;
    p.ws_rows = static_cast<int64_t>(num_seqs) * num_q_heads * p.num_parts;
    p.ws = static_cast<float *>(workspace);
    p.num_seqs = num_seqs;
    p.head_dim = head_dim;
    p.ws_bytes = workspace ? workspace_bytes : 0;
    return p;
}

}  // namespace

int launch_reduce(const AttnParams &p, int32_t dtype, int32_t head_dim, int32_t num_seqs, hipStream_t stream) {
#define PKV_RED(E, D) hipLaunchKernelGGL((attn_reduce_kernel<E, D>), dim3(p.num_q_heads, num_seqs), dim3(D), 0, stream, p)
    switch (dtype * 1000 + head_dim) {
    case PKV_F32 * 1000 + 64: PKV_RED(F32, 64); break;
    case PKV_F32 * 1000 + 128: PKV_RED(F32, 128); break;
    case PKV_F16 * 1000 + 64: PKV_RED(F16, 64); break;
    case PKV_F16 * 1000 + 128: PKV_RED(F16, 128); break;
    case PKV_BF16 * 1000 + 64: PKV_RED(BF16, 64); break;
    case PKV_BF16 * 1000 + 128: PKV_RED(BF16, 128); break;
    default: return fail(PKV_EUNSUPPORTED, "reduce: dtype %d head_dim %d not built", dtype, head_dim);
    }
#undef PKV_RED
    return hip_status(hipGetLastError(), "attention reduce launch");
}

int launch_reduce_balanced(const AttnParams &p, int32_t dtype, int32_t head_dim, hipStream_t stream) {
#define PKV_RED(E, D) \
    hipLaunchKernelGGL((attn_reduce_balanced_kernel<E, D>), dim3(p.balanced_wgs), dim3(256), 0, stream, p)
    switch (dtype * 1000 + head_dim) {
    case PKV_F32 * 1000 + 64: PKV_RED(F32, 64); break;
    case PKV_F32 * 1000 + 128: PKV_RED(F32, 128); break;
    case PKV_F16 * 1000 + 64: PKV_RED(F16, 64); break;
    case PKV_F16 * 1000 + 128: PKV_RED(F16, 128); break;
    case PKV_BF16 * 1000 + 64: PKV_RED(BF16, 64); break;
    case PKV_BF16 * 1000 + 128: PKV_RED(BF16, 128); break;
    default: return fail(PKV_EUNSUPPORTED, "reduce: dtype %d head_dim %d not built", dtype, head_dim);
    }
#undef PKV_RED
    return hip_status(hipGetLastError(), "balanced reduce launch");
}

int device_compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int balanced_check(AttnParams &p, int wgs_per_cu) {
    if (p.num_seqs > kBalancedMaxSeqs)
        return fail(PKV_EUNSUPPORTED, "balanced partitioning: %d sequences, at most %d", p.num_seqs, kBalancedMaxSeqs);
    const int64_t tiles = static_cast<int64_t>(p.num_seqs) * ceil_div(p.ctx_cap, p.tile_rows);
    if (tiles >= (int64_t(1) << 31)) return fail(PKV_EINVAL, "balanced partitioning: %lld tiles per row", (long long)tiles);
    const int cus = device_compute_units();
    if (cus <= 0) return fail(PKV_EHIP, "balanced partitioning: cannot read the device's compute-unit count");
    p.balanced_wgs = wgs_per_cu * cus;
    const size_t need = static_cast<size_t>(2) * p.balanced_wgs * p.heads_per_row * (p.head_dim + 2) * sizeof(float) +
                        (kBalancedMaxSeqs + 1) * sizeof(uint32_t) + static_cast<size_t>(2) * p.balanced_wgs * sizeof(int32_t);
    if (!p.ws || p.ws_bytes < need)
        return fail(PKV_EINVAL, "balanced partitioning: workspace of %zu bytes needed, %zu given", need, p.ws_bytes);
    return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t partition_size) {
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
    if (partition_size == PKV_PARTITION_BALANCED) {
        // two partial-result slots per workgroup, each for up to num_q_heads heads
        const int cus = device_compute_units();
        if (cus <= 0) return 0;
        return static_cast<size_t>(2) * kBalancedWgsPerCu * cus * num_q_heads * (head_dim + 2) * sizeof(float) +
               (kBalancedMaxSeqs + 1) * sizeof(uint32_t) + static_cast<size_t>(2) * kBalancedWgsPerCu * cus * sizeof(int32_t);
    }
    if (partition_size <= 0) return 0;
    const int64_t parts = ceil_div(max_context_len, partition_size);
    const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads * parts;
    const int cus = device_compute_units();
    if (head_dim == 128 && num_q_heads >= 2 && cus > 0) {
        // room for the grouped-query kernel's persistent schedule, for any group it may serve
        const int64_t group = std::min<int64_t>(num_q_heads, kGqaMaxGroup);
        return parts_workspace_bytes(rows, head_dim, parts_slot_count(cus, group),
                                     static_cast<int64_t>(num_seqs) * num_q_heads);
    }
    return static_cast<size_t>(rows) * (head_dim + 2) * sizeof(float);
}

namespace pkv {
namespace {

// The paged decode entry points: attention alone (new_k == nullptr), or a decode step that also
// writes each sequence's new key and value rows to their slots in the same launch.
int paged_decode(const char *fn, void *out, const void *q, const void *k_cache, const void *v_cache,
                 int64_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                 const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale, int32_t partition_size,
                 void *workspace, size_t workspace_bytes, int32_t dtype, uint32_t flags, const int32_t *cached_lens,
                 const void *new_k, const void *new_v, const int64_t *slot_mapping, void *k_write, void *v_write,
                 hipStream_t stream) {
    int rc = check_common(fn, out, q, k_cache, v_cache, context_lens, max_context_len, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, scale, partition_size, workspace, workspace_bytes, dtype);
    if (rc || num_seqs == 0) return rc;
    if (flags & ~(PKV_FLAG_SCALAR_GQA | PKV_FLAG_CACHED_KV)) return fail(PKV_EINVAL, "%s: unknown flags %#x", fn, flags);
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EUNSUPPORTED, "%s: block_size %d not built (8, 16, 32)", fn, block_size);
    if (partition_size > 0 && partition_size % block_size)
        return fail(PKV_EINVAL, "%s: partition_size %d is not a multiple of block_size %d", fn, partition_size,
                    block_size);
    if (!block_tables || max_blocks_per_seq <= 0 || num_blocks <= 0)
        return fail(PKV_EINVAL, "%s: block_tables NULL or max_blocks_per_seq / num_blocks not positive", fn);
    if (num_blocks > INT32_MAX) return fail(PKV_EINVAL, "%s: num_blocks %lld exceeds int32", fn, (long long)num_blocks);
    if (new_k && (!new_v || !slot_mapping || !aligned16(new_k) || !aligned16(new_v)))
        return fail(PKV_EINVAL, "%s: new_k, new_v (16-byte aligned) and slot_mapping are needed", fn);
    if (debug_validate()) {
        rc = validate_attention(fn, context_lens, num_seqs, max_context_len, block_tables, max_blocks_per_seq,
                                block_size, num_blocks, 0, stream);
        if (!rc && cached_lens && !(flags & PKV_FLAG_CACHED_KV))
            rc = validate_device_array(fn, "cached_lens", cached_lens);
        if (!rc && new_k)
            rc = validate_step_slots(fn, slot_mapping, context_lens, block_tables, num_seqs, max_blocks_per_seq,
                                     block_size, stream);
        if (rc) return rc;
    }
    const int64_t cap = std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * block_size);
    AttnParams p = make_params(out, q, k_cache, v_cache, context_lens, num_seqs, num_q_heads, num_kv_heads, scale,
                               partition_size, max_context_len, static_cast<int32_t>(cap), workspace,
                               workspace_bytes, head_dim);
    p.tables = block_tables;
    p.cached_lens = cached_lens;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = static_cast<uint32_t>(num_blocks);
    p.new_k = new_k;
    p.new_v = new_v;
    p.new_slots = slot_mapping;
    p.num_slots = num_blocks * block_size;
    p.k_write = k_write;
    p.v_write = v_write;
    const int32_t grid_parts = p.partition_size > 0 ? static_cast<int32_t>(ceil_div(cap, p.partition_size)) : 1;
    if (new_k && p.group > 1 && !(flags & PKV_FLAG_SCALAR_GQA) &&
        gqa_mfma_supported(dtype, head_dim, block_size, p.group)) {
        // the grouped-query matrix-core path writes the new rows with its own launch first (one
        // launch measured slower there: the substitution sits in its matrix-core loop), then
        // attends over the cache that holds them
        rc = pkv_reshape_and_cache(new_k, new_v, static_cast<int64_t>(num_kv_heads) * head_dim,
                                   static_cast<int64_t>(num_kv_heads) * head_dim, k_write, v_write, num_blocks,
                                   slot_mapping, num_seqs, num_kv_heads, head_dim, block_size, dtype, stream);
        if (rc) return rc;
        p.new_k = p.new_v = nullptr;
        p.new_slots = nullptr;
    }
    return dispatch<true>(p, dtype, head_dim, block_size, num_seqs, grid_parts, flags, stream);
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                                          int64_t num_blocks, const int32_t *block_tables,
                                          int32_t max_blocks_per_seq, const int32_t *context_lens,
                                          int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                                          int32_t partition_size, void *workspace, size_t workspace_bytes,
                                          int32_t dtype, uint32_t flags, const int32_t *cached_lens,
                                          hipStream_t stream) {
    return paged_decode("pkv_paged_attention_decode", out, q, k_cache, v_cache, num_blocks, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads,
                        head_dim, block_size, scale, partition_size, workspace, workspace_bytes, dtype, flags,
                        cached_lens, nullptr, nullptr, nullptr, nullptr, nullptr, stream);
}

extern "C" int pkv_paged_attention_decode_step(void *out, const void *q, const void *new_k, const void *new_v,
                                               const int64_t *slot_mapping, void *k_cache, void *v_cache,
                                               int64_t num_blocks, const int32_t *block_tables,
                                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                                               int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                               float scale, int32_t partition_size, void *workspace,
                                               size_t workspace_bytes, int32_t dtype, uint32_t flags,
                                               const int32_t *cached_lens, hipStream_t stream) {
    const char *fn = "pkv_paged_attention_decode_step";
    if (num_seqs > 0 && (!new_k || !new_v || !slot_mapping)) return fail(PKV_EINVAL, "%s: NULL pointer", fn);
    return paged_decode(fn, out, q, k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq, context_lens,
                        max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                        partition_size, workspace, workspace_bytes, dtype, flags, cached_lens, new_k, new_v,
                        slot_mapping, k_cache, v_cache, stream);
}

extern "C" int pkv_contiguous_attention_decode(void *out, const void *q, const void *k, const void *v, int32_t lmax,
                                               const int32_t *context_lens, int32_t max_context_len,
                                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, float scale, int32_t partition_size,
                                               void *workspace, size_t workspace_bytes, int32_t dtype,
                                               uint32_t flags, hipStream_t stream) {
    const char *fn = "pkv_contiguous_attention_decode";
    int rc = check_common(fn, out, q, k, v, context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads,
                          head_dim, scale, partition_size, workspace, workspace_bytes, dtype);
    if (rc || num_seqs == 0) return rc;
    if (flags & ~(PKV_FLAG_SCALAR_GQA | PKV_FLAG_CACHED_KV)) return fail(PKV_EINVAL, "%s: unknown flags %#x", fn, flags);
    if (lmax <= 0) return fail(PKV_EINVAL, "%s: lmax must be positive", fn);
    // tile rows of the contiguous slab: 16 (any multiple of rows-per-load works)
    constexpr int32_t kTile = 16;
    if (partition_size > 0 && partition_size % kTile) return fail(PKV_EINVAL, "%s: partition_size must be a multiple of 16", fn);
    if (debug_validate()) {
        rc = validate_attention(fn, context_lens, num_seqs, max_context_len, nullptr, 0, 0, 0, lmax, stream);
        if (rc) return rc;
    }
    const int32_t cap = std::min(max_context_len, lmax);
    AttnParams p = make_params(out, q, k, v, context_lens, num_seqs, num_q_heads, num_kv_heads, scale,
                               partition_size, max_context_len, cap, workspace, workspace_bytes, head_dim);
    p.lmax = lmax;
    const int32_t grid_parts = p.partition_size > 0 ? static_cast<int32_t>(ceil_div(cap, p.partition_size)) : 1;
    return dispatch<false>(p, dtype, head_dim, kTile, num_seqs, grid_parts, flags, stream);
}

// ---------------------------------------------------------------- no-allocation decode
// The split workspace of pkv_paged_attention_decode_noalloc: one static array per device, held
// until the process ends. Host code never passes `scratch` itself to a kernel (on the host that
// name is a stand-in, not a device address): it passes the address hipGetSymbolAddress gives
// for the current device, looked up once per device.
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace pkv {
namespace {

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device (PKV_OK), or an error.
int scratch_address(void **out) {
    static std::atomic<void *> cache[kMaxDevices];
    static std::mutex setup;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKV_EHIP, "pkv_paged_attention_decode_noalloc: no current HIP device");
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKV_EUNSUPPORTED, "pkv_paged_attention_decode_noalloc: device %d (at most %d devices)", dev,
                    kMaxDevices);
    void *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(setup);
        p = cache[dev].load(std::memory_order_relaxed);
        if (!p) {
            const int rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                                      "pkv_paged_attention_decode_noalloc: address of the static scratch");
            if (rc) return rc;
            if (!p) return fail(PKV_EHIP, "pkv_paged_attention_decode_noalloc: the static scratch has no address");
            cache[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_paged_attention_decode_noalloc(void *out, const void *q, const void *k_cache,
                                                  const void *v_cache, int64_t num_blocks,
                                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                                  const int32_t *context_lens, int32_t max_context_len,
                                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t block_size, float scale,
                                                  int32_t partition_size, int32_t dtype, uint32_t flags,
                                                  const int32_t *cached_lens, hipStream_t stream) {
    const char *fn = "pkv_paged_attention_decode_noalloc";
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (partition_size != 0 && num_seqs > 0) {
        // the size rule of the caller-provided workspace, checked against the static array first
        const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size);
        if (need > PKV_NOALLOC_SCRATCH_BYTES)
            return fail(PKV_EINVAL, "%s: the split needs %zu bytes of workspace, the static scratch holds %zu", fn, need,
                        static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES));
        if (need > 0) {
            const int rc = scratch_address(&ws);
            if (rc) return rc;
            ws_bytes = PKV_NOALLOC_SCRATCH_BYTES;
        }
    }
    return paged_decode(fn, out, q, k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq, context_lens,
                        max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                        partition_size, ws, ws_bytes, dtype, flags, cached_lens, nullptr, nullptr, nullptr, nullptr,
                        nullptr, stream);
}
