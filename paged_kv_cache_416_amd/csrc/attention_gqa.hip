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
constexpr int kGqaStages = 2;  // stages in flight + the one consumed

template <int W>
struct GqaLds {
    float m[W][kGqaMaxGroup], l[W][kGqaMaxGroup];
    float acc[W][kGqaMaxGroup][128];
    u32x4 kt[W][16 * 16];  // each wave's K tile, 16 rows x 16 chunks, chunk positions swizzled by row
};


// One 16-row tile's contribution to the running softmax state (max m, weight sum lsum, Oᵀ
// accumulators) of the group's heads. kr / vr: the tile's K and V rows as loaded (load i: chunk
// n of row 4g + i); rows 0 .. rows - 1 count, the rest are masked out (rows <= 0: none). The K
// rows reach the A-operand layout through the wave's LDS tile kt (a wave's LDS operations
// complete in order, so the reads see the writes and the next tile's writes follow them).
template <class E>
__device__ inline void gqa_tile(const u32x4 (&kr)[4], const u32x4 (&vr)[4], const u32x4 (&qv)[4], int rows,
                                float scale_log2, u32x4 *kt, float &m, float &lsum, f32x4 (&acc)[8]) {
    using M = Mfma<E>;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;
    // K operand: chunk c of row r at position c ^ r of the row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        kt[r * 16 + (n ^ r)] = kr[i];
    }
    u32x4 ka[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ka[kk] = kt[n * 16 + ((4 * kk + g) ^ n)];
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) c = M::mma(ka[kk], qv[kk], c);
    float sc[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sc[i] = 4 * g + i < rows ? c[i] * scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, sc[i]);
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
    // P^T operand: head n, tokens 4g .. 4g+3. The matrix cores take 16-bit operands, so each
    // weight goes in as a 16-bit part plus the 16-bit rounding of its remainder (the remainder of
    // a round to nearest is exact in fp32): two contractions see the fp32 weight to about 2^-16
    // relative. The sum l takes the same parts (a dot2 with (1, 1) per pair).
    const float e0 = fast_exp2(sc[0] - m_ref), e1 = fast_exp2(sc[1] - m_ref);
    const float e2 = fast_exp2(sc[2] - m_ref), e3 = fast_exp2(sc[3] - m_ref);
    const unsigned h01 = M::pack2(e0, e1), h23 = M::pack2(e2, e3);
    const unsigned r01 = M::pack2(e0 - M::value(h01 & 0xffffu), e1 - M::value(h01 >> 16));
    const unsigned r23 = M::pack2(e2 - M::value(h23 & 0xffffu), e3 - M::value(h23 >> 16));
    lsum = M::sum2(r23, M::sum2(r01, M::sum2(h23, M::sum2(h01, lsum))));
    const u32x2 ph = {h01, h23}, pr = {r01, r23};
    // (a masked row reads as zeros and its weight is zero)
    // V^T operand of MFMA j: element j of the lane's 4 V rows
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = j >> 1;
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
        const u32x2 vt = {__builtin_amdgcn_perm(word(vr[1], w), word(vr[0], w), sel),
                          __builtin_amdgcn_perm(word(vr[3], w), word(vr[2], w), sel)};
        acc[j] = M::mma16(vt, pr, M::mma16(vt, ph, acc[j]));
    }
    m = m_new;
}

// Tokens [t0, t1) of sequence s for kv head kvh and its G query heads (t0 a multiple of 16,
// t0 < t1 <= the length): the workgroup's merged result goes to sink. Uniform over the
// workgroup; ends with a barrier, so the caller may run it again on the same LDS. head_dim 128,
// 16-bit types.
//
// The range's tiles go to the waves round-robin, one tile a stage. Each wave keeps NS stages in
// registers: while it consumes one, the next NS - 1 are in flight, and the table entry of the
// stage after those is on the way.
template <class E, int B, bool PAGED, int W, int POL>
__device__ inline void gqa_range(const AttnParams &p, int s, int kvh, int t0, int t1, const Sink &sink,
                                 GqaLds<W> &lds) {
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

    // the next tile this wave will issue (wave w takes tiles w, w + W, w + 2W, ...: a fixed
    // assignment, so the summation order and the result do not depend on timing) and its table
    // entry, looked up one stage ahead
    int cst = wave;
    int cpb = 0;
    auto lookup = [&]() {
        const int k = min(cst, ntile - 1);  // a stand-in past the range reads the last entry
        cpb = PAGED ? trow[(jt0 + k) / SPB] : 0;
    };
    lookup();

    struct Stage {
        u32x4 k[4], v[4];  // [i]: chunk n of row 4g + i
        int st;   // tile index within the range (>= ntile: a stand-in)
        bool ok;  // table entry inside the pool
    };

    // Every load is unconditional (exact wait counts) and goes through a buffer resource that
    // ends at the tile's last row inside [t0, t1): rows past it, a stand-in tile and a tile whose
    // table entry is rejected read as zeros, with no memory traffic; the tile update masks them.
    const unsigned roff = g * 4 * ROWB + n * 16;  // + i * ROWB: row 4g + i, chunk n (K and V)
    auto issue = [&](Stage &S) {
        S.st = cst;
        const int jt = jt0 + min(cst, ntile - 1);
        int64_t tile;
        if constexpr (PAGED) {
            S.ok = static_cast<uint32_t>(cpb) < p.num_blocks;  // 32-bit, so it stays a scalar compare
            const int64_t blk = S.ok ? cpb : 0;
            tile = ((blk * p.num_kv_heads + kvh) * B + (jt % SPB) * TR) * ROWB;
        } else {
            S.ok = true;
            tile = ((static_cast<int64_t>(s) * p.num_kv_heads + kvh) * p.lmax + static_cast<int64_t>(jt) * TR) * ROWB;
        }
        const int rows = cst < ntile && S.ok ? min(TR, t1 - (jt0 + cst) * TR) : 0;
        const auto kr_ = tile_rsrc(kc + tile, rows * ROWB), vr_ = tile_rsrc(vc + tile, rows * ROWB);
        if (POL == kLoadCached || (POL == kLoadSplit && (jt0 + cst) * TR < clen)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S.k[i] = kv_buffer_load<false>(kr_, roff + i * ROWB);
#pragma unroll
            for (int i = 0; i < 4; ++i) S.v[i] = kv_buffer_load<false>(vr_, roff + i * ROWB);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) S.k[i] = kv_buffer_load<true>(kr_, roff + i * ROWB);
#pragma unroll
            for (int i = 0; i < 4; ++i) S.v[i] = kv_buffer_load<true>(vr_, roff + i * ROWB);
        }
        cst += W;
        lookup();
    };

    float m = -INFINITY, lsum = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 *kt = lds.kt[wave];
    auto consume = [&](Stage &S) {
        // a stand-in's rows all lie past t1
        const int rows = S.ok ? t1 - (jt0 + S.st) * TR : 0;
        gqa_tile<E>(S.k, S.v, qv, rows, p.scale_log2, kt, m, lsum, acc);
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
        if (R[0].st >= ntile) break;
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
template <class E, int B, bool PAGED, int W, int POL>
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
    gqa_range<E, B, PAGED, W, POL>(p, s, kvh, t0, t1, sink, lds);
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
template <class E, int B, bool PAGED, int W, int POL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_gqa_balanced_kernel(
    const AttnParams p) {
    __shared__ GqaLds<W> lds;
    __shared__ uint32_t C[kBalancedMaxSeqs + 1];
    __shared__ uint32_t part[W * 64];
    balanced_prefix<W * 64>(p, C, part, balanced_prefix_out(p));
    balanced_zero_empty<E, 128, W * 64>(p, C);
    balanced_walk<128, true>(p, C, [&](int s, int kvh, int ta, int tb, const Sink &sink) {
        const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
        gqa_range<E, B, PAGED, W, POL>(p, s, kvh, ta * 16, min(tb * 16, ctx), sink, lds);
    });
}

// Fixed partitions on a persistent schedule: grid = balanced_wgs workgroups (one per CU) of
// kGqaPartsWaves waves, and every wave of the grid takes an equal share of the balanced
// schedule's tile list (work rows = (kv head, sequence), head-major; each XCD a contiguous run
// of shares). A wave streams its share through one register ring, across partition and row
// boundaries, with no barrier: no wave waits for another. The tiles of one partition inside one
// share form a piece, computed on its own. A piece that starts at its partition's start belongs
// to the partition's workspace row, as on the per-item grid; any other piece starts at its
// wave's share start (a share boundary cut the partition) and belongs to the wave's slot. A
// finished piece goes to the workgroup's LDS pool, not to memory. After the workgroup's last
// barrier, rows whose pieces all sit in the pool are merged there and written to the output,
// and the pieces of the other rows go to the workspace for the merge pass.

// Where head j of a finished piece goes: its destination code c is the partition row of the
// group's head 0 (c >= 0; head j at row c + j * num_parts) or -(w + 1) for wave w's slot.
__device__ inline void piece_dest(const AttnParams &p, int64_t c, int j, float *&pa, float *&pm, float *&pl) {
    constexpr int D = 128;
    if (c < 0) {
        float *sl = p.ws + parts_slot_offset(p.ws_rows, D);
        const int64_t nsl = parts_slot_count(p.balanced_wgs, p.group), r = (-c - 1) * p.group + j;
        pa = sl + r * D;
        pm = sl + nsl * D + r;
        pl = sl + nsl * (D + 1) + r;
    } else {
        const int64_t r = c + static_cast<int64_t>(j) * p.num_parts;
        pa = p.ws + r * D;
        pm = p.ws + p.ws_rows * D + r;
        pl = p.ws + p.ws_rows * (D + 1) + r;
    }
}

// The workgroup's LDS pool of finished pieces: piece b is acc [G][128], m [G], l [G] at
// piece + b * G * 130, with its destination code, first tile and work row beside it. A wave
// claims a piece with an LDS atomic (`used` may pass cap: a piece that finds the pool full is
// stored at once). The pool is emptied after the workgroup's last barrier.
struct PiecePool {
    float *piece;
    int64_t *dst;     // destination code
    int32_t *key;     // wave * 65536 + the piece's index among the wave's pieces (tile order);
                      // cap + 1 entries
    int32_t *row;     // its work row (kv head * num_seqs + sequence)
    int32_t *order;   // the pieces in tile order (filled after the last wave is done)
    uint32_t *used;
    uint32_t cap;
    int32_t *nruns;   // after the last wave: runs of pieces of one row
    uint32_t *need;   // per wave of the workgroup: while streaming, the tiles it has yet to request
                      // (its SIMD partner levels against it); after the last wave, whether its
                      // slot is written neutral
    uint32_t *count;  // per wave of the workgroup: its pieces
    int32_t *first_row;  // the first work row that starts in the workgroup's tiles (from wave 0's
                         // share), or -1 when wave 0's share is empty
};

// Where a wave's share starts: the row holding its first tile (none for an empty share), and
// whether that tile starts one of the row's partitions.
struct ShareHead {
    bool has = false;
    bool starts_row = false;
    bool starts_part = false;
    int r = 0;         // work row: kv head * num_seqs + sequence
    int nrow = 0;      // the row's tiles
    int64_t row0 = 0;  // its first tile's list position
};

// Returns the number of pieces the wave finished (uniform).
template <class E, int B, bool PAGED, int POL, int QL>
__device__ inline int gqa_share(const AttnParams &p, const uint32_t *C, int64_t v, int64_t nw, u32x4 *kt,
                                const PiecePool &pool, ShareHead &head) {
    constexpr int D = 128;
    constexpr int TR = 16;
    constexpr int SPB = B / TR;
    constexpr int ROWB = D * 2;
    static_assert(B % TR == 0, "block_size must be a multiple of 16");

    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;
    const int G = p.group, S_ = p.num_seqs, PT = p.partition_size / TR;
    const int64_t Ctot = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(C[S_]));
    const int64_t T = Ctot * p.num_kv_heads;
    const int64_t xb = balanced_begin(v, T, nw), xe = balanced_begin(v + 1, T, nw);
    // a wave's slot, neutral: the merge pass may read it when the wave has no cut piece
    auto neutral_slot = [&]() {
        for (int c = lane; c < G * 32; c += 64) {
            float *pa, *pm, *pl;
            piece_dest(p, -(v + 1), c >> 5, pa, pm, pl);
            *reinterpret_cast<f32x4 *>(pa + (c & 31) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
            if ((c & 31) == 0) {
                *pm = -INFINITY;
                *pl = 0.f;
            }
        }
    };
    if (xb >= xe) {
        neutral_slot();
        return 0;
    }

    // The issue cursor, all uniform: the next tile x; its row (sequence s, kv head kvh, first
    // position row0, nrow tiles, ctx tokens, clen of them through the caches); its partition
    // (index part in the row, positions [pbeg, pend)); its table entry. Partition boundaries
    // advance by additions: only a share's first tile divides.
    int64_t x = xb, row0 = 0, pbeg = 0, pend = 0;
    int s = 0, kvh = 0, nrow = 0, ctx = 0, clen = 0, cpb = 0, part = 0;
    TableEntry *trow = nullptr;
    auto locate = [&]() {
        kvh = static_cast<int>(x / Ctot);
        const int64_t rem = x - kvh * Ctot;
        int lo = 0, hi = S_;  // the largest lo with C[lo] <= rem, which has tiles (C[lo + 1] > rem)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(C[mid])) <= rem) lo = mid; else hi = mid;
        }
        s = lo;
        const uint32_t c0 = __builtin_amdgcn_readfirstlane(C[s]);
        row0 = kvh * Ctot + c0;
        nrow = static_cast<int>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(C[s + 1])) - c0);
        ctx = clamp_ctx(*(TableEntry *)(p.ctx_lens + s), p.ctx_cap);  // scalar loads, like the table's
        clen = POL == kLoadSplit ? *(TableEntry *)(p.cached_lens + s) : 0;
        if constexpr (PAGED) trow = (TableEntry *)(p.tables + static_cast<int64_t>(s) * p.max_blocks);
        part = 0;
        if (x != row0) part = static_cast<int>((x - row0) / PT);
        pbeg = row0 + static_cast<int64_t>(part) * PT;
        pend = min(row0 + nrow, pbeg + PT);
    };
    auto lookup = [&]() {
        if constexpr (PAGED) cpb = trow[static_cast<int>(x - row0) / SPB];
    };
    locate();
    lookup();
    head.has = true;
    head.starts_row = x == row0;
    head.starts_part = x == pbeg;
    head.r = kvh * S_ + s;
    head.nrow = nrow;
    head.row0 = row0;

    struct Stage {
        u32x4 k[4], v[4];  // [i]: chunk n of row 4g + i
        u32x4 q[QL];       // the group's query rows (16 bytes a lane each), loaded for a piece's
                           // first tile (zeros otherwise)
        int64_t dst;       // the partition's workspace row for the group's head 0
        int rowid;         // its work row: kvh * num_seqs + s
        int rows;          // rows of the tile that count (0: none)
        bool valid;        // a tile of the share (else a stand-in past its end)
        bool first, last;  // the first / last tile of a piece
        bool slot;         // (first) the piece goes to the wave's slot
    };

    // Every load is unconditional (exact wait counts) and goes through a buffer resource that
    // ends at the tile's last counted row: rows past it, a stand-in and a rejected table entry
    // read as zeros with no memory traffic, and the query loads of a tile that starts no piece
    // move nothing.
    const unsigned roff = g * 4 * ROWB + n * 16;  // + i * ROWB: row 4g + i, chunk n (K and V)
    // the query loads: QL = ceil(G / 4) of them (16 bytes a lane, 1 KiB each), so that a tile
    // adds few load instructions; the operand layout is made through LDS at a piece's first tile
    auto issue = [&](Stage &S) {
        const bool valid = x < xe;
        const int jt = static_cast<int>(x - row0);
        const int64_t row_q0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(kvh) * G;
        S.valid = valid;
        S.dst = row_q0 * p.num_parts + part;
        S.rowid = kvh * S_ + s;
        S.first = valid && (x == xb || x == pbeg);
        S.slot = x == xb && x != pbeg;
        S.last = valid && (x + 1 == xe || x + 1 == pend);
        int64_t tile;
        bool ok;
        if constexpr (PAGED) {
            ok = static_cast<uint32_t>(cpb) < p.num_blocks;  // 32-bit, so it stays a scalar compare
            const int64_t blk = ok ? cpb : 0;
            tile = ((blk * p.num_kv_heads + kvh) * B + (jt % SPB) * TR) * ROWB;
        } else {
            ok = true;
            tile = ((static_cast<int64_t>(s) * p.num_kv_heads + kvh) * p.lmax + static_cast<int64_t>(jt) * TR) * ROWB;
        }
        const int rows = valid && ok ? min(TR, ctx - jt * TR) : 0;
        S.rows = rows;
        const auto kr_ = tile_rsrc(static_cast<const char *>(p.k) + tile, rows * ROWB);
        const auto vr_ = tile_rsrc(static_cast<const char *>(p.v) + tile, rows * ROWB);
        if (POL == kLoadCached || (POL == kLoadSplit && jt * TR < clen)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S.k[i] = kv_buffer_load<false>(kr_, roff + i * ROWB);
#pragma unroll
            for (int i = 0; i < 4; ++i) S.v[i] = kv_buffer_load<false>(vr_, roff + i * ROWB);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) S.k[i] = kv_buffer_load<true>(kr_, roff + i * ROWB);
#pragma unroll
            for (int i = 0; i < 4; ++i) S.v[i] = kv_buffer_load<true>(vr_, roff + i * ROWB);
        }
        const auto qr_ = tile_rsrc(static_cast<const char *>(p.q) + row_q0 * ROWB, S.first ? G * ROWB : 0);
#pragma unroll
        for (int u = 0; u < QL; ++u) S.q[u] = kv_buffer_load<false>(qr_, (u * 64 + lane) * 16);
        if (valid) {
            ++x;
            if (x < xe) {
                if (x == row0 + nrow) {
                    locate();
                } else if (x == pend) {
                    ++part;
                    pbeg = x;
                    pend = min(row0 + nrow, x + PT);
                }
                lookup();
            }
        }
    };

    u32x4 qv[4];  // the current piece's query operand
    float m = -INFINITY, lsum = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool to_slot = false;
    int prow = 0;        // the current piece's work row
    int npieces = 0;     // pieces finished so far

    // A piece's result, unnormalised (acc, m, l of each of the G heads), into the workgroup's
    // pool, written out after the last barrier: a store in the stream would hold up the wave's
    // later loads until it is acknowledged, which under a saturated memory system takes about a
    // full queue drain. Then the state starts over for the next piece.
    auto finish = [&](const Stage &S) {
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        const int64_t code = to_slot ? -(v + 1) : S.dst;
        uint32_t b = 0;
        if (lane == 0) b = atomicAdd(pool.used, 1u);
        b = __builtin_amdgcn_readfirstlane(b);
        // lane (n, g) holds d = 8 (4g + i) + j: columns 32g .. 32g + 31 of head n
        if (b < pool.cap) {
            float *pc = pool.piece + static_cast<int64_t>(b) * G * (D + 2);
            if (n < G) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 *dst = reinterpret_cast<f32x4 *>(pc + n * D + 8 * (4 * g + i));
                    dst[0] = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
                    dst[1] = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
                }
                if (g == 0) {
                    pc[G * D + n] = m;
                    pc[G * (D + 1) + n] = lsum;
                }
            }
            if (lane == 0) {
                pool.dst[b] = code;
                pool.key[b] = static_cast<int32_t>(threadIdx.x >> 6) * 65536 + npieces;
                pool.row[b] = prow;
            }
        } else if (n < G) {
            float *pa, *pm, *pl;
            piece_dest(p, code, n, pa, pm, pl);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 *dst = reinterpret_cast<f32x4 *>(pa + 8 * (4 * g + i));
                dst[0] = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
                dst[1] = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
            }
            if (g == 0) {
                *pm = m;
                *pl = lsum;
            }
        }
        m = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        ++npieces;
    };

    auto consume = [&](Stage &S) {
        if (S.first) {
            // the rows through the wave's LDS tile (the tile is free between two consumes), read
            // back as the operand: query head n, chunks 4 * kk + g; zero for n >= G
#pragma unroll
            for (int u = 0; u < QL; ++u) kt[u * 64 + lane] = S.q[u];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qv[kk] = n < G ? kt[n * 16 + 4 * kk + g] : u32x4{0u, 0u, 0u, 0u};
            to_slot = S.slot;
            prow = S.rowid;
        }
        gqa_tile<E>(S.k, S.v, qv, S.rows, p.scale_log2, kt, m, lsum, acc);
        if (S.last) finish(S);
    };

    // A ring of two stages: while one is consumed the other is in flight.
    // The two waves of a SIMD (w and w ^ 4) keep level: each publishes the tiles it has yet to
    // request, and the one with more left runs at raised priority. The SIMD's issue arbitration
    // otherwise serves the older wave first, and the younger one ends well after it. The room of
    // the pool's per-wave flags is free until the drain.
    const int me = static_cast<int>(v & (kGqaPartsWaves - 1));
    Stage R[2];
    issue(R[0]);
    __builtin_amdgcn_sched_barrier(0);
    for (;;) {
        if (!R[0].valid) break;
        const uint32_t mine = static_cast<uint32_t>(xe - x);
        pool.need[me] = mine;
        const uint32_t other = pool.need[me ^ 4];
        issue(R[1]);
        consume(R[0]);
        if (mine > other)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        issue(R[0]);
        consume(R[1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    return npieces;
}

// LDS of the persistent schedule: the waves' K tiles, the prefix sums C, then the piece pool.
constexpr int kPartsLdsBytes = 160 * 1024;
constexpr int kPartsKtBytes = kGqaPartsWaves * 16 * 16 * 16;

// After the workgroup's last wave is done: the pool's pieces in tile order (a wave's pieces are
// in tile order and the waves' shares follow one another, so a piece's place is the count of
// the earlier waves' pieces plus its index). A work row whose tiles all lie in this
// workgroup's tiles [X0, X1), with every piece in the pool, is merged here (the partitions'
// merge, in tile order) and written to the output; the pieces of any other row go to the
// workspace for the merge pass. flags[row] records which, for every row that starts in
// [X0, X1); a wave of this workgroup whose share starts a partition of a row left to the merge
// pass gets a neutral slot. The LDS work comes first, behind LDS-only barriers; every global
// write comes after the last barrier (a block barrier would also wait for stores to complete).
template <class E>
__device__ inline void parts_drain(const AttnParams &p, const uint32_t *C, const PiecePool &pool, int64_t vw0,
                                   int64_t nw, int32_t *flags, const ShareHead &head) {
    using M = Mfma<E>;
    constexpr int D = 128;
    constexpr int NT = kGqaPartsWaves * 64;
    constexpr int NB = 8;  // pieces whose loads are in flight together while a row is merged
    const int G = p.group, S = p.num_seqs;
    const int64_t Ctot = C[S], T = Ctot * p.num_kv_heads;
    const int64_t X0 = balanced_begin(vw0, T, nw), X1 = balanced_begin(vw0 + kGqaPartsWaves, T, nw);
    const uint32_t used = *pool.used, np = min(used, pool.cap);
    const bool spilled = used > pool.cap;  // pieces were stored at once: no row is merged here
    if (X0 >= X1) return;
    // the row holding list position x (0 <= x < T)
    auto locate = [&](int64_t x, int &r, int64_t &row0, int &nrow) {
        const int kvh = static_cast<int>(x / Ctot);
        const int64_t rem = x - kvh * Ctot;
        int lo = 0, hi = S;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (C[mid] <= rem) lo = mid; else hi = mid;
        }
        r = kvh * S + lo;
        row0 = kvh * Ctot + C[lo];
        nrow = static_cast<int>(C[lo + 1] - C[lo]);
    };
    auto merged = [&](int64_t row0, int nrow) { return !spilled && row0 >= X0 && row0 + nrow <= X1; };
    auto lds_barrier = [] {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
    };
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // tile order (unused when spilled: every piece then goes to the workspace)
    if (!spilled)
        for (int b = threadIdx.x; b < static_cast<int>(np); b += NT) {
            const int w = pool.key[b] >> 16;
            int base = 0;
            for (int w2 = 0; w2 < w; ++w2) base += pool.count[w2];
            pool.order[base + (pool.key[b] & 0xffff)] = b;
        }
    // the waves whose shares start a partition of a row that the merge pass takes (each wave's own
    // share start, as its stream found it)
    if (lane == 0) pool.need[wave] = head.has && head.starts_part && !merged(head.row0, head.nrow);
    lds_barrier();
    // runs of pieces of one row, in order: their first places (the keys' room is free now), each
    // tagged kRunMerged when its row is merged here
    constexpr int kRunMerged = 1 << 30;
    int32_t *runs = pool.key;
    if (wave == 0) {
        int nr = 0;
        for (int base = 0; base < static_cast<int>(np); base += 64) {
            const int i = base + lane;
            const int b = spilled ? i : pool.order[i < static_cast<int>(np) ? i : 0];
            const int bp = spilled ? i - 1 : pool.order[i > 0 && i < static_cast<int>(np) ? i - 1 : 0];
            const bool st = i < static_cast<int>(np) && (i == 0 || pool.row[b] != pool.row[bp]);
            const uint64_t m = __builtin_amdgcn_ballot_w64(st);
            if (st) {
                const int r = pool.row[b], kvh = r / S, s = r - kvh * S;
                const bool mg = merged(kvh * Ctot + C[s], static_cast<int>(C[s + 1] - C[s]));
                runs[nr + __builtin_popcountll(m & ((uint64_t(1) << lane) - 1))] = i | (mg ? kRunMerged : 0);
            }
            nr += __builtin_popcountll(m);
        }
        if (lane == 0) {
            runs[nr] = static_cast<int>(np);
            *pool.nruns = nr;
        }
    }
    lds_barrier();

    // flags of the rows that start here
    {
        int r0 = *pool.first_row;
        if (r0 < 0) {  // wave 0's share is empty: the row holding X0, unless it starts earlier
            int64_t row0;
            int nrow;
            locate(X0, r0, row0, nrow);
            if (row0 < X0) ++r0;
        }
        for (int r = r0 + threadIdx.x; r < p.num_kv_heads * S; r += NT) {
            const int kvh = r / S, s = r - kvh * S;
            const int64_t rs = kvh * Ctot + C[s];
            if (rs >= X1) break;
            flags[r] = merged(rs, static_cast<int>(C[s + 1] - C[s])) ? 1 : 0;
        }
    }
    for (int c = threadIdx.x; c < kGqaPartsWaves * G * 32; c += NT) {
        const int w = c / (G * 32), cc = c - w * G * 32;
        if (!pool.need[w]) continue;
        float *pa, *pm, *pl;
        piece_dest(p, -(vw0 + w + 1), cc >> 5, pa, pm, pl);
        *reinterpret_cast<f32x4 *>(pa + (cc & 31) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
        if ((cc & 31) == 0) {
            *pm = -INFINITY;
            *pl = 0.f;
        }
    }
    // A row merged here goes to the output, the rows one per wave in turn (a row's merge is one
    // chain over its pieces). Any other row's pieces go to the workspace, shared out over all the
    // waves, a piece per wave in turn: copied by one wave, a cut row of tens of pieces held up the
    // workgroup's end by microseconds. A lane holds 16 bytes (4 columns of one head). The runs'
    // entries are read 63 at a time, one a lane.
    const int nruns = *pool.nruns;
    auto at = [&](int i) { return spilled ? i : pool.order[i]; };
    for (int kb = 0; kb < nruns; kb += 63) {
        const int ent = runs[min(kb + lane, nruns)];
        const int kn = min(63, nruns - kb);
        for (int kk = 0; kk < kn; ++kk) {
            const int e0 = __builtin_amdgcn_readlane(ent, kk), e1 = __builtin_amdgcn_readlane(ent, kk + 1);
            const int i0 = e0 & ~kRunMerged, i1 = e1 & ~kRunMerged;
            if (e0 & kRunMerged) {
                if ((kb + kk) % kGqaPartsWaves != wave) continue;
                const int r = pool.row[at(i0)];
                const int kvh = r / S, s = r - kvh * S;
                const int64_t row_q0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(kvh) * G;
                // two column chunks a lane (c0 and c0 + 64) in one pass: their pieces' places are read
                // once, and both chains of loads are in flight together
                auto add = [](float &M, float &L, f32x4 &O, float mg, float lg, const f32x4 &og) {
                    const float Mn = fmaxf(M, mg);
                    const float Mr = Mn == -INFINITY ? 0.f : Mn;
                    const float a = fast_exp2(M - Mr), f = fast_exp2(mg - Mr);
                    L = fmaf(lg, f, L * a);
#pragma unroll
                    for (int e = 0; e < 4; ++e) O[e] = fmaf(og[e], f, O[e] * a);
                    M = Mn;
                };
                // four outputs, each O / L as the merge pass takes it, in one 8-byte store
                auto put = [&](int c, float L, const f32x4 &O) {
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = L > 0.f ? O[e] / L : 0.f;
                    const u32x2 packed = {M::pack2(o[0], o[1]), M::pack2(o[2], o[3])};
                    const int64_t at_out = ((row_q0 + (c >> 5)) * D + (c & 31) * 4) * 2;
                    *reinterpret_cast<u32x2 *>(static_cast<char *>(p.out) + at_out) = packed;
                };
                for (int c0 = lane; c0 < G * 32; c0 += 128) {
                    const int c1 = c0 + 64;
                    const bool has1 = c1 < G * 32;
                    const int h0 = c0 >> 5, h1 = has1 ? c1 >> 5 : h0;
                    float M0 = -INFINITY, L0 = 0.f, M1 = -INFINITY, L1 = 0.f;
                    f32x4 O0 = {0.f, 0.f, 0.f, 0.f}, O1 = {0.f, 0.f, 0.f, 0.f};
                    for (int t0 = i0; t0 < i1; t0 += NB) {
                        int bb[NB];
#pragma unroll
                        for (int u = 0; u < NB; ++u) bb[u] = pool.order[min(t0 + u, i1 - 1)];
                        float mg0[NB], lg0[NB], mg1[NB], lg1[NB];
                        f32x4 og0[NB], og1[NB];
#pragma unroll
                        for (int u = 0; u < NB; ++u) {
                            const float *pc = pool.piece + static_cast<int64_t>(bb[u]) * G * (D + 2);
                            mg0[u] = pc[G * D + h0];
                            lg0[u] = pc[G * (D + 1) + h0];
                            og0[u] = *reinterpret_cast<const f32x4 *>(pc + c0 * 4);
                            mg1[u] = pc[G * D + h1];
                            lg1[u] = pc[G * (D + 1) + h1];
                            og1[u] = *reinterpret_cast<const f32x4 *>(pc + (has1 ? c1 : c0) * 4);
                        }
#pragma unroll
                        for (int u = 0; u < NB; ++u) {
                            if (t0 + u < i1) {
                                add(M0, L0, O0, mg0[u], lg0[u], og0[u]);
                                add(M1, L1, O1, mg1[u], lg1[u], og1[u]);
                            }
                        }
                    }
                    put(c0, L0, O0);
                    if (has1) put(c1, L1, O1);
                }
            } else {
                // copied four pieces at a time, so that their LDS reads are in flight together (one
                // chunk after another, each a chain of lookups, reads and a store, took microseconds
                // for the rows of tens of pieces)
                constexpr int NC = 4;
                // this wave's pieces: i0 + wave + kGqaPartsWaves t, t < n
                const int n = (i1 - i0 - wave + kGqaPartsWaves - 1) / kGqaPartsWaves;
                for (int t0 = 0; t0 < n; t0 += NC) {
                    int b[NC];
                    int64_t code[NC];
#pragma unroll
                    for (int u = 0; u < NC; ++u) b[u] = at(i0 + wave + kGqaPartsWaves * min(t0 + u, n - 1));
#pragma unroll
                    for (int u = 0; u < NC; ++u) code[u] = pool.dst[b[u]];
                    for (int cc = lane; cc < G * 32; cc += 64) {
                        const int hj = cc >> 5;
                        f32x4 o[NC];
                        float mv[NC], lv[NC];
#pragma unroll
                        for (int u = 0; u < NC; ++u) {
                            const float *pc = pool.piece + static_cast<int64_t>(b[u]) * G * (D + 2);
                            o[u] = *reinterpret_cast<const f32x4 *>(pc + cc * 4);
                            mv[u] = pc[G * D + hj];
                            lv[u] = pc[G * (D + 1) + hj];
                        }
#pragma unroll
                        for (int u = 0; u < NC; ++u) {
                            if (t0 + u < n) {
                                float *pa, *pm, *pl;
                                piece_dest(p, code[u], hj, pa, pm, pl);
                                *reinterpret_cast<f32x4 *>(pa + (cc & 31) * 4) = o[u];
                                if ((cc & 31) == 0) {
                                    *pm = mv[u];
                                    *pl = lv[u];
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

template <class E, int B, bool PAGED, int POL, int QL>
__global__ __launch_bounds__(kGqaPartsWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_gqa_parts_kernel(
    const AttnParams p) {
    constexpr int D = 128;
    constexpr int NT = kGqaPartsWaves * 64;
    __shared__ __attribute__((aligned(16))) char smem[kPartsLdsBytes];
    const int G = p.group;
    const int cbytes = ((p.num_seqs + 1) * 4 + 15) / 16 * 16;
    uint32_t *C = reinterpret_cast<uint32_t *>(smem + kPartsKtBytes);
    char *rest = smem + kPartsKtBytes + cbytes;
    // the pool: an 80-byte header (counter, run count, per-wave flags and piece counts, the first
    // row), then
    // dst [cap], key [cap + 1] (the runs share its room), row [cap], order [cap], then the pieces,
    // 16-byte aligned
    static_assert(2 + 2 * kGqaPartsWaves + 1 <= 20, "the pool header: two counters, two words a wave, the first row");
    const uint32_t cap = static_cast<uint32_t>((kPartsLdsBytes - kPartsKtBytes - cbytes - 112) / (G * (D + 2) * 4 + 20));
    char *q0 = rest + 80;
    const PiecePool pool{reinterpret_cast<float *>(q0 + (cap * 20 + 4 + 15) / 16 * 16), reinterpret_cast<int64_t *>(q0),
                         reinterpret_cast<int32_t *>(q0 + cap * 8), reinterpret_cast<int32_t *>(q0 + cap * 12 + 4),
                         reinterpret_cast<int32_t *>(q0 + cap * 16 + 4), reinterpret_cast<uint32_t *>(rest), cap,
                         reinterpret_cast<int32_t *>(rest + 4), reinterpret_cast<uint32_t *>(rest + 8),
                         reinterpret_cast<uint32_t *>(rest + 8 + 4 * kGqaPartsWaves),
                         reinterpret_cast<int32_t *>(rest + 8 + 8 * kGqaPartsWaves)};
    if (threadIdx.x == 0) *pool.used = 0u;
    if (threadIdx.x < kGqaPartsWaves) pool.need[threadIdx.x] = 0xffffffffu;  // no progress published yet
    // the prefix scan's scratch sits where the pool will be (its last use precedes its last barrier)
    const int64_t slots = parts_slot_count(p.balanced_wgs, G);
    uint32_t *prefix = reinterpret_cast<uint32_t *>(p.ws + parts_prefix_offset(p.ws_rows, D, slots));
    balanced_prefix<NT>(p, C, reinterpret_cast<uint32_t *>(q0), prefix);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nw = static_cast<int64_t>(p.balanced_wgs) * kGqaPartsWaves;
    const int64_t vw0 = balanced_virtual(blockIdx.x, p.balanced_wgs) * kGqaPartsWaves;
    ShareHead head;
    const int npieces = gqa_share<E, B, PAGED, POL, QL>(p, C, vw0 + wave, nw,
                                                        reinterpret_cast<u32x4 *>(smem) + wave * 256, pool, head);
    if ((threadIdx.x & 63) == 0) {
        pool.count[wave] = npieces;
        if (wave == 0) *pool.first_row = head.has ? head.r + (head.starts_row ? 0 : 1) : -1;
    }
    __syncthreads();
    parts_drain<E>(p, C, pool, vw0, nw, reinterpret_cast<int32_t *>(prefix + kBalancedMaxSeqs + 1), head);
}

// The merge pass of the persistent schedule, for the rows the attention kernel left to it (its
// flags): grid = (num_kv_heads, num_seqs), one lane per 4 adjacent columns of the group's G heads
// (G x 32 lanes), one pass with a running maximum over the row's partitions (their workspace
// rows), then over the slots of the waves whose shares begin inside the row (owner of its first
// tile < w <= owner of its last: a cut piece of one of its partitions, or neutral). The share
// boundaries depend only on the tile count. The work is a chain of dependent loads (the flags,
// then the pieces), so the lanes take all their columns in one pass, with 16-byte loads and 16
// pieces in flight at a time.
template <class E>
__global__ __launch_bounds__(kGqaMaxGroup * 32) void attn_gqa_reduce_parts_kernel(const AttnParams p) {
    constexpr int D = 128;
    constexpr int TR = 16;
    constexpr int NB = 16;
    const int kvh = blockIdx.x, s = blockIdx.y, G = p.group;
    const int64_t nsl = parts_slot_count(p.balanced_wgs, G);
    const float *sl = p.ws + parts_slot_offset(p.ws_rows, D);
    const uint32_t *C = reinterpret_cast<const uint32_t *>(p.ws + parts_prefix_offset(p.ws_rows, D, nsl));
    // the three prefix sums first, so that their loads are in flight together
    const uint32_t c0 = C[s], c1 = C[s + 1], cS = C[p.num_seqs];
    const int32_t done = reinterpret_cast<const int32_t *>(C + kBalancedMaxSeqs + 1)[kvh * p.num_seqs + s];
    const int64_t Ctot = cS, T = Ctot * p.num_kv_heads;
    const int64_t nw = static_cast<int64_t>(p.balanced_wgs) * kGqaPartsWaves;
    const int PT = p.partition_size / TR;
    const int64_t row0 = kvh * Ctot + c0;
    const int nrow = static_cast<int>(c1 - c0);
    const int c = threadIdx.x;
    if ((nrow > 0 && done) || c >= G * 32) return;  // merged by the attention kernel; a lane past the group
    const int np = (nrow + PT - 1) / PT;
    const int64_t w0 = nrow > 0 ? balanced_owner(row0, T, nw) + 1 : 0;
    const int64_t w1 = nrow > 0 ? balanced_owner(row0 + nrow - 1, T, nw) : -1;
    const int64_t row_q0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(kvh) * G;
    const int j = c >> 5, d4 = (c & 31) * 4;
    float M = -INFINITY, L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    const int64_t wr = (row_q0 + j) * p.num_parts;
    const int total = np + static_cast<int>(w1 - w0 + 1);
    for (int t0 = 0; t0 < total; t0 += NB) {
        float mg[NB], lg[NB];
        f32x4 og[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int t = t0 + u;
            mg[u] = -INFINITY;
            lg[u] = 0.f;
            og[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < total) {
                const bool row = t < np;
                const int64_t r = row ? wr + t : (w0 + t - np) * G + j;
                const float *base = row ? p.ws : sl;
                const int64_t rows = row ? p.ws_rows : nsl;
                mg[u] = base[rows * D + r];
                lg[u] = base[rows * (D + 1) + r];
                og[u] = *reinterpret_cast<const f32x4 *>(base + r * D + d4);
            }
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (t0 + u < total) {  // a guard, not a break: the loop unrolls and the pieces stay in registers
                const float Mn = fmaxf(M, mg[u]);
                const float Mr = Mn == -INFINITY ? 0.f : Mn;
                const float a = fast_exp2(M - Mr), f = fast_exp2(mg[u] - Mr);
                L = fmaf(lg[u], f, L * a);
#pragma unroll
                for (int e = 0; e < 4; ++e) O[e] = fmaf(og[u][e], f, O[e] * a);
                M = Mn;
            }
        }
    }
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = L > 0.f ? O[e] / L : 0.f;
    const u32x2 packed = {Mfma<E>::pack2(o[0], o[1]), Mfma<E>::pack2(o[2], o[3])};
    *reinterpret_cast<u32x2 *>(static_cast<char *>(p.out) + ((row_q0 + j) * D + d4) * 2) = packed;
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
        hipLaunchKernelGGL((attn_gqa_balanced_kernel<E, B, PAGED, kGqaBalancedWaves, POL>),
                           dim3(q.balanced_wgs), dim3(kGqaBalancedWaves * 64), 0, stream, q);
        rc = hip_status(hipGetLastError(), "grouped-query attention launch");
        return rc ? rc : launch_reduce_balanced(q, E::CODE, 128, stream);
    }
    if (p.partition_size > 0) {
        // fixed partitions: the persistent schedule where its limits and workspace allow
        AttnParams q = p;
        q.tile_rows = 16;
        q.rows_per_seq = p.num_kv_heads;
        q.heads_per_row = p.group;
        q.head_major = 1;
        const int cus = device_compute_units();
        const int64_t tiles = static_cast<int64_t>(num_seqs) * ceil_div(p.ctx_cap, 16) * p.num_kv_heads;
        if (cus > 0 && num_seqs <= kBalancedMaxSeqs && tiles < (int64_t(1) << 31) && q.ws &&
            q.ws_bytes >= parts_workspace_bytes(q.ws_rows, 128, parts_slot_count(cus, q.group),
                                                static_cast<int64_t>(num_seqs) * p.num_kv_heads)) {
            q.balanced_wgs = cus;
            if (q.group <= 4)
                hipLaunchKernelGGL((attn_gqa_parts_kernel<E, B, PAGED, POL, 1>), dim3(cus), dim3(kGqaPartsWaves * 64),
                                   0, stream, q);
            else if (q.group <= 8)
                hipLaunchKernelGGL((attn_gqa_parts_kernel<E, B, PAGED, POL, 2>), dim3(cus), dim3(kGqaPartsWaves * 64),
                                   0, stream, q);
            else
                hipLaunchKernelGGL((attn_gqa_parts_kernel<E, B, PAGED, POL, 4>), dim3(cus), dim3(kGqaPartsWaves * 64),
                                   0, stream, q);
            int rc = hip_status(hipGetLastError(), "grouped-query attention launch");
            if (rc) return rc;
            hipLaunchKernelGGL((attn_gqa_reduce_parts_kernel<E>), dim3(p.num_kv_heads, num_seqs),
                               dim3((q.group * 32 + 63) / 64 * 64), 0, stream, q);
            return hip_status(hipGetLastError(), "grouped-query reduce launch");
        }
    }
    hipLaunchKernelGGL((attn_gqa_mfma_kernel<E, B, PAGED, kGqaWaves, POL>),
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
           group >= 2 && group <= kGqaMaxGroup;
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
