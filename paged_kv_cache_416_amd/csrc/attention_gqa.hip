// Grouped-query decode attention on the matrix cores: the G query heads that share one
// KV head are served by one workgroup, so each K/V tile is read from HBM once, and both
// contractions run on MFMA.
//
// Same result as the one-head-per-workgroup kernel: single-query scaled dot-product attention
// of each query head over its sequence's keys and values, gathered block by block through the
// block table ("vLLM and PagedAttention" slide 9 and slide 10). Query head h reads KV head
// h / G.
//
// Work unit: a tile of 16 consecutive rows (tokens) of one (block, kv head). With lane l,
// g = l / 16, n = l % 16:
//  * K and V are loaded alike, as whole rows: load i brings lane l chunk n of row 4g + i, so one
//    load instruction covers four whole 256-byte rows and every 128-byte line is fetched by one
//    instruction (which lets the loads be non-temporal without fetching a line twice);
//  * logits: S^T[token][head] = K[token][:] . Q^T[:][head] as 4 v_mfma_f32_16x16x32 over d.
//    Lane l supplies K row n, 16-byte chunk 4*kk + g (the A operand) and query head n, the same
//    chunk (the B operand; heads >= G are zero), and receives the logits of head n for tokens
//    4g .. 4g+3 of the tile. The K tile reaches that operand layout through a 4 KiB LDS tile
//    private to the wave: written as loaded, read back per operand, with chunk c of row r stored
//    at position c ^ r of the row, so that neither the 16 lanes writing one row nor the 16 lanes
//    reading one chunk of 16 rows meet in a bank;
//  * weighted sum: O^T[d][head] = V^T[d][token] . P^T[token][head] as 8 v_mfma_f32_16x16x16,
//    MFMA j covering d = 8m + j (m = 0..15). Lane l's P^T operand is its own 4 softmax
//    weights (head n, tokens 4g .. 4g+3) and its V^T operand is element j of its own 4 V loads
//    (rows 4g .. 4g+3, chunk n), packed in pairs with v_perm: no value crosses lanes between
//    the two contractions;
//  * the output tile leaves head n and d = 8(4g + i) + j in lane l, so the online-softmax
//    rescale of a head is lane-local; only the running max crosses the four lane groups, and
//    the rescale is skipped when no head's max moved.
// The softmax weights enter the second contraction as two 16-bit parts each (the rounded
// weight and its rounded remainder), so that contraction sees them to about 2^-16 relative,
// and the sum l is taken over the same parts.
// Loads, table handling, double buffering, masking and the split workspace are as in the
// one-head kernel. The grid is (kv heads, partitions, sequences) with the kv head fastest, so a
// kv head's workgroups land on the same XCDs and a shared prefix stays in their L2.
#include "attention.h"
#include "mfma.h"

namespace pkv {
namespace {

constexpr int kGqaWaves = 4;          // per-item schedule: two workgroups per CU
constexpr int kGqaBalancedWaves = 8;  // balanced schedule: one workgroup per CU (two waves per SIMD)
constexpr int kGqaTiles = 1;   // tiles per stage
constexpr int kGqaStages = 2;  // stages in flight + the one consumed
constexpr int kMaxGroup = 16;

template <int W>
struct GqaLds {
    float m[W][kMaxGroup], l[W][kMaxGroup];
    float acc[W][kMaxGroup][128];
    u32x4 kt[W][16 * 16];  // each wave's K tile, 16 rows x 16 chunks, chunk positions swizzled by row
};


// Tokens [t0, t1) of sequence s for kv head kvh and its G query heads (t0 a multiple of 16,
// t0 < t1 <= the length): the workgroup's merged result goes to sink. Uniform over the
// workgroup; ends with a barrier, so the caller may run it again on the same LDS. head_dim 128,
// 16-bit types.
//
// The range's tiles go to the waves in stages of U tiles, round-robin. Each wave keeps NS
// stages in registers: while it consumes one, the next NS - 1 are in flight, and the table
// entries of the stage after those are on the way.
template <class E, int B, bool PAGED, int W, int U, int POL>
__device__ inline void gqa_range(const AttnParams &p, int s, int kvh, int t0, int t1, const Sink &sink,
                                 GqaLds<W> &lds) {
    using M = Mfma<E>;
    constexpr int D = 128;
    constexpr int TR = 16;          // tile rows
    constexpr int SPB = B / TR;     // tiles per block
    constexpr int ROWB = D * 2;     // bytes per row
    constexpr int NS = kGqaStages;
    static_assert(B % TR == 0, "block_size must be a multiple of 16");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers, scalar branches
    const int G = p.group;
    const int n = lane & 15, g = lane >> 4;
    const int jt0 = t0 / TR;
    const int ntile = (t1 + TR - 1) / TR - jt0;
    const int nstage = (ntile + U - 1) / U;
    const int64_t row_q0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(kvh) * G;
    TableEntry *trow = PAGED ? (TableEntry *)(p.tables + static_cast<int64_t>(s) * p.max_blocks)  // address-space cast
                             : nullptr;

    // Q^T operand: query head n of the group, chunks 4*kk + g; zero for n >= G.
    u32x4 qv[4];
    {
        const char *qp = static_cast<const char *>(p.q) + ((row_q0 + n) * D + g * 8) * 2;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qv[kk] = n < G ? *reinterpret_cast<const u32x4 *>(qp + kk * 64) : u32x4{0u, 0u, 0u, 0u};
    }

    const char *kc = static_cast<const char *>(p.k);
    const char *vc = static_cast<const char *>(p.v);
    // tokens below clen are loaded through the caches (uniform: a scalar compare per tile)
    const int clen = POL == kLoadSplit ? __builtin_amdgcn_readfirstlane(p.cached_lens[s]) : 0;

    // the next stage this wave will issue (wave w takes stages w, w + W, w + 2W, ...: a fixed
    // assignment, so the summation order and the result do not depend on timing) and its
    // table entries, looked up one stage ahead
    int cst = wave;
    int cpb[U];
    auto lookup = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = min(cst * U + u, ntile - 1);  // a stand-in past the range reads the last entry
            cpb[u] = PAGED ? trow[(jt0 + k) / SPB] : 0;
        }
    };
    lookup();

    struct Stage {
        u32x4 k[U][4], v[U][4];  // [i]: chunk n of row 4g + i
        int st;      // stage index within the range (>= nstage: a stand-in)
        bool ok[U];  // table entry inside the pool
    };

    // Every load is unconditional (exact wait counts) and goes through a buffer resource that
    // ends at the tile's last row inside [t0, t1): rows past it, a stand-in tile and a tile whose
    // table entry is rejected read as zeros, with no memory traffic; consume() masks them out.
    const unsigned roff = g * 4 * ROWB + n * 16;  // + i * ROWB: row 4g + i, chunk n (K and V)
    auto issue = [&](Stage &S) {
        S.st = cst;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = cst * U + u;
            const int jt = jt0 + min(k, ntile - 1);
            int64_t tile;
            if constexpr (PAGED) {
                S.ok[u] = static_cast<uint32_t>(cpb[u]) < p.num_blocks;  // 32-bit, so it stays a scalar compare
                const int64_t blk = S.ok[u] ? cpb[u] : 0;
                tile = ((blk * p.num_kv_heads + kvh) * B + (jt % SPB) * TR) * ROWB;
            } else {
                S.ok[u] = true;
                tile = ((static_cast<int64_t>(s) * p.num_kv_heads + kvh) * p.lmax + static_cast<int64_t>(jt) * TR) * ROWB;
            }
            const int rows = k < ntile && S.ok[u] ? min(TR, t1 - (jt0 + k) * TR) : 0;
            const auto kr_ = tile_rsrc(kc + tile, rows * ROWB), vr_ = tile_rsrc(vc + tile, rows * ROWB);
            if (POL == kLoadCached || (POL == kLoadSplit && (jt0 + k) * TR < clen)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) S.k[u][i] = kv_buffer_load<false>(kr_, roff + i * ROWB);
#pragma unroll
                for (int i = 0; i < 4; ++i) S.v[u][i] = kv_buffer_load<false>(vr_, roff + i * ROWB);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) S.k[u][i] = kv_buffer_load<true>(kr_, roff + i * ROWB);
#pragma unroll
                for (int i = 0; i < 4; ++i) S.v[u][i] = kv_buffer_load<true>(vr_, roff + i * ROWB);
            }
        }
        cst += W;
        lookup();
    };

    float m = -INFINITY, lsum = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The K tile in the A-operand layout: through the wave's LDS tile (a wave's LDS operations
    // complete in order, so a tile's reads see its writes and the next tile's writes follow them).
    u32x4 *kt = lds.kt[wave];
    auto k_operand = [&](const u32x4 (&rows)[4], u32x4 (&ka)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            kt[r * 16 + (n ^ r)] = rows[i];
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[kk] = kt[n * 16 + ((4 * kk + g) ^ n)];
    };

    auto consume = [&](Stage &S) {
        float sc[U][4];
        float mloc = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 ka[4];
            k_operand(S.k[u], ka);
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) c = M::mma(ka[kk], qv[kk], c);
            const int tok0 = (jt0 + S.st * U + u) * TR;  // a stand-in's rows all lie past t1
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = S.ok[u] && tok0 + 4 * g + i < t1;
                sc[u][i] = valid ? c[i] * p.scale_log2 : -INFINITY;
                mloc = fmaxf(mloc, sc[u][i]);
            }
        }
        // the head's running max over its four lane groups (lanes n, n+16, n+32, n+48)
        mloc = max_over_lane_groups(mloc);
        const float m_new = fmaxf(m, mloc);
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        // rescale only when some head's max moved: rare after the first tiles (uniform branch)
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(m_new > m) != 0, 0)) {
            const float alpha = fast_exp2(m - m_ref);
            lsum *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // P^T operand: head n, tokens 4g .. 4g+3 of tile u. The matrix cores take 16-bit
            // operands, so each weight goes in as a 16-bit part plus the 16-bit rounding of its
            // remainder (the remainder of a round to nearest is exact in fp32): two contractions
            // see the fp32 weight to about 2^-16 relative. The sum l takes the same parts (a dot2
            // with (1, 1) per pair).
            const float e0 = fast_exp2(sc[u][0] - m_ref), e1 = fast_exp2(sc[u][1] - m_ref);
            const float e2 = fast_exp2(sc[u][2] - m_ref), e3 = fast_exp2(sc[u][3] - m_ref);
            const unsigned h01 = M::pack2(e0, e1), h23 = M::pack2(e2, e3);
            const unsigned r01 = M::pack2(e0 - M::value(h01 & 0xffffu), e1 - M::value(h01 >> 16));
            const unsigned r23 = M::pack2(e2 - M::value(h23 & 0xffffu), e3 - M::value(h23 >> 16));
            lsum = M::sum2(r23, M::sum2(r01, M::sum2(h23, M::sum2(h01, lsum))));
            const u32x2 ph = {h01, h23}, pr = {r01, r23};
            // (a rejected or stand-in tile reads as zeros and its weights are zero)
            // V^T operand of MFMA j: element j of the lane's 4 V rows
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = j >> 1;
                const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const u32x2 vt = {__builtin_amdgcn_perm(word(S.v[u][1], w), word(S.v[u][0], w), sel),
                                  __builtin_amdgcn_perm(word(S.v[u][3], w), word(S.v[u][2], w), sel)};
                acc[j] = M::mma16(vt, pr, M::mma16(vt, ph, acc[j]));
            }
        }
        m = m_new;
    };

    // A ring of NS stages; the wave stops once the oldest stage is past the range (its later
    // stages are stand-ins too).
    Stage R[NS];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
        issue(R[i]);  // in order: the first stage's loads return first
        __builtin_amdgcn_sched_barrier(0);
    }
    // Whole rounds of NS stages, the test for the end only at a round's start: straight-line
    // rounds keep the compiler's wait counts exact. The last round may consume up to NS - 1
    // stand-ins (zeros, masked; their loads move no data).
    for (;;) {
        if (R[0].st >= nstage) break;
#pragma unroll
        for (int r = 0; r < NS; ++r) {
            issue(R[(r + NS - 1) % NS]);
            consume(R[r]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // the head's weight sum over the four lane groups (each holds its own tokens' share)
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (n < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) lds.acc[wave][n][8 * (4 * g + i) + j] = acc[j][i];
        if (g == 0) {
            lds.m[wave][n] = m;
            lds.l[wave][n] = lsum;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += W * 64) {
        const int h = idx / D, dd = idx % D;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) Mx = fmaxf(Mx, lds.m[w][h]);
        const float Mr = Mx == -INFINITY ? 0.f : Mx;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = fast_exp2(lds.m[w][h] - Mr);
            L = fmaf(lds.l[w][h], f, L);
            O = fmaf(lds.acc[w][h][dd], f, O);
        }
        if (sink.acc) {
            sink.acc[h * sink.acc_stride + dd] = O;
            if (dd == 0) {
                sink.m[h * sink.ml_stride] = Mx;
                sink.l[h * sink.ml_stride] = L;
            }
        } else {
            E::store(p.out, (row_q0 + h) * D + dd, L > 0.f ? O / L : 0.f);
        }
    }
    __syncthreads();
}

// Per-item schedule: grid = (num_kv_heads, parts, num_seqs), block = 64 * W, the kv head fastest
// so that a kv head's workgroups share XCDs (and the L2 holding a shared prefix). At most 256
// registers per lane (two waves per SIMD): two workgroups share a CU and one's start-up hides
// behind the other.
template <class E, int B, bool PAGED, int W, int U, int POL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_gqa_mfma_kernel(
    const AttnParams p) {
    __shared__ GqaLds<W> lds;
    const int kvh = blockIdx.x, part = blockIdx.y, s = blockIdx.z;
    const int G = p.group;
    const int64_t row_q0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(kvh) * G;
    const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
    const int t0 = p.partition_size > 0 ? part * p.partition_size : 0;
    const int t1 = p.partition_size > 0 ? min(ctx, t0 + p.partition_size) : ctx;
    if (t0 >= t1) {
        if (p.partition_size == 0)
            for (int i = threadIdx.x; i < G * 128; i += W * 64) E::store(p.out, row_q0 * 128 + i, 0.f);
        return;
    }
    Sink sink{nullptr, nullptr, nullptr, 0, 0};
    if (p.partition_size > 0) {
        const int64_t wr = row_q0 * p.num_parts + part;  // head j: workspace row wr + j * num_parts
        sink = Sink{p.ws + wr * 128, p.ws + p.ws_rows * 128 + wr, p.ws + p.ws_rows * 129 + wr,
                    static_cast<int64_t>(p.num_parts) * 128, p.num_parts};
    }
    gqa_range<E, B, PAGED, W, U, POL>(p, s, kvh, t0, t1, sink, lds);
}

// The fixed-partition merge of one (sequence, kv head): grid = (num_kv_heads, num_seqs), the kv
// head fastest like the attention grid, so a workgroup reads the partials its XCD's L2 received;
// 256 threads over the group's G heads x 128 columns. One pass over the partitions with a
// running maximum (the partitions' loads are independent):
//   M = max_p m_p, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
template <class E>
__global__ __launch_bounds__(256) void attn_gqa_reduce_kernel(const AttnParams p) {
    constexpr int D = 128;
    const int kvh = blockIdx.x, s = blockIdx.y, G = p.group;
    const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
    const int np = (ctx + p.partition_size - 1) / p.partition_size;
    const int64_t row_q0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(kvh) * G;
    for (int i = threadIdx.x; i < G * D; i += 256) {
        const int j = i / D, d = i % D;
        const int64_t wr = (row_q0 + j) * p.num_parts;
        const float *wacc = p.ws + wr * D + d;
        const float *wm = p.ws + p.ws_rows * D + wr;
        const float *wl = p.ws + p.ws_rows * (D + 1) + wr;
        float M = -INFINITY, L = 0.f, O = 0.f;
#pragma unroll 4
        for (int k = 0; k < np; ++k) {
            const float mg = wm[k], lg = wl[k], og = wacc[static_cast<int64_t>(k) * D];
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

// Balanced schedule: grid = balanced_wgs workgroups (one per CU), each an equal share of the
// batch's tiles (work rows = (kv head, sequence), head-major); cut rows are merged by the
// balanced reduce pass. One workgroup per CU because two sharing a CU do not progress at one
// pace (the older one's waves are served first), and the later one would finish alone.
template <class E, int B, bool PAGED, int W, int U, int POL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_gqa_balanced_kernel(
    const AttnParams p) {
    __shared__ GqaLds<W> lds;
    __shared__ uint32_t C[kBalancedMaxSeqs + 1];
    __shared__ uint32_t part[W * 64];
    balanced_prefix<W * 64>(p, C, part);
    balanced_zero_empty<E, 128, W * 64>(p, C);
    balanced_walk<128, true>(p, C, [&](int s, int kvh, int ta, int tb, const Sink &sink) {
        const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
        gqa_range<E, B, PAGED, W, U, POL>(p, s, kvh, ta * 16, min(tb * 16, ctx), sink, lds);
    });
}

template <class E, int B, bool PAGED, int POL>
int launch_one(const AttnParams &p, int32_t num_seqs, int32_t grid_parts, hipStream_t stream) {
    if (p.partition_size == PKV_PARTITION_BALANCED) {
        AttnParams q = p;
        q.tile_rows = 16;
        q.rows_per_seq = p.num_kv_heads;
        q.heads_per_row = p.group;
        q.head_major = 1;  // an XCD's shares cover few kv heads: shared blocks stay in its L2
        int rc = balanced_check(q, 1);  // one workgroup per CU: two per CU would not run at one pace
        if (rc) return rc;
        hipLaunchKernelGGL((attn_gqa_balanced_kernel<E, B, PAGED, kGqaBalancedWaves, kGqaTiles, POL>),
                           dim3(q.balanced_wgs), dim3(kGqaBalancedWaves * 64), 0, stream, q);
        rc = hip_status(hipGetLastError(), "grouped-query attention launch");
        return rc ? rc : launch_reduce_balanced(q, E::CODE, 128, stream);
    }
    hipLaunchKernelGGL((attn_gqa_mfma_kernel<E, B, PAGED, kGqaWaves, kGqaTiles, POL>),
                       dim3(p.num_kv_heads, grid_parts, num_seqs), dim3(kGqaWaves * 64), 0, stream, p);
    int rc = hip_status(hipGetLastError(), "grouped-query attention launch");
    if (rc || p.partition_size <= 0) return rc;
    hipLaunchKernelGGL((attn_gqa_reduce_kernel<E>), dim3(p.num_kv_heads, num_seqs), dim3(256), 0, stream, p);
    return hip_status(hipGetLastError(), "grouped-query reduce launch");
}

template <class E, int B>
int launch_policy(const AttnParams &p, int pol, int32_t num_seqs, int32_t grid_parts, hipStream_t stream) {
    if (pol == kLoadCached) return launch_one<E, B, true, kLoadCached>(p, num_seqs, grid_parts, stream);
    if (pol == kLoadSplit) return launch_one<E, B, true, kLoadSplit>(p, num_seqs, grid_parts, stream);
    return launch_one<E, B, true, kLoadStream>(p, num_seqs, grid_parts, stream);
}

template <class E, bool PAGED>
int launch_block(const AttnParams &p, int32_t block_size, int pol, int32_t num_seqs, int32_t grid_parts,
                 hipStream_t stream) {
    if constexpr (!PAGED) {
        return launch_one<E, 16, false, kLoadStream>(p, num_seqs, grid_parts, stream);  // 16-row tiles
    } else {
        return block_size == 32 ? launch_policy<E, 32>(p, pol, num_seqs, grid_parts, stream)
                                : launch_policy<E, 16>(p, pol, num_seqs, grid_parts, stream);
    }
}

}  // namespace

bool gqa_mfma_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
    return (dtype == PKV_F16 || dtype == PKV_BF16) && head_dim == 128 && (block_size == 16 || block_size == 32) &&
           group >= 2 && group <= kMaxGroup;
}

int launch_gqa_mfma(const AttnParams &p, int32_t dtype, int32_t block_size, bool paged, int load_policy,
                    int32_t num_seqs, int32_t grid_parts, hipStream_t stream) {
    if (p.num_kv_heads > 65535 || grid_parts > 65535)
        return fail(PKV_EINVAL, "grouped-query attention: %d kv heads x %d partitions exceed the grid", p.num_kv_heads,
                    grid_parts);
    if (dtype == PKV_F16)
        return paged ? launch_block<F16, true>(p, block_size, load_policy, num_seqs, grid_parts, stream)
                     : launch_block<F16, false>(p, block_size, load_policy, num_seqs, grid_parts, stream);
    return paged ? launch_block<BF16, true>(p, block_size, load_policy, num_seqs, grid_parts, stream)
                 : launch_block<BF16, false>(p, block_size, load_policy, num_seqs, grid_parts, stream);
}

}  // namespace pkv
