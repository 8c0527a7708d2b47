// Prefill (chunked) attention over the paged cache on the matrix cores: each sequence's last n_s
// tokens are queries, and query i (at position p = ctx - n_s + i) attends causally to the keys at
// positions 0 .. p, earlier chunks and shared prefix blocks included ("vLLM and PagedAttention"
// slide 3: the prompt is processed in parallel; slides 9 and 10: keys and values are fetched
// block by block through the block table).
//
// The grouped-query decode kernel's tile generalised: a wave owns 16 matrix rows, now (query
// token, query head) pairs of one kv head (row r of a sequence and kv head is token r / G, head
// kvh * G + r % G), and walks every 16-key tile up to its last row's position:
//  * logits: S^T[key][row] = K[key][:] . Q^T[:][row] as 4 v_mfma_f32_16x16x32 over d;
//  * weighted sum: O^T[d][row] = V^T[d][key] . P^T[key][row] as 8 v_mfma_f32_16x16x16 per
//    16-bit part of the weights (each weight enters as a 16-bit part and the 16-bit rounding
//    of its remainder), lane-local operands as in the decode kernel;
//  * the causal mask is a per-lane compare of the key's position with row n's position.
// Rows are independent, so the waves of a workgroup (consecutive row tiles, reading the same
// key tiles through the caches) need no merge; a wave writes its rows and ends.
#include "mfma.h"

namespace pkv {
namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillStages = 2;
constexpr int kPrefillRowTiles = 2;  // 16-row tiles per wave, sharing each key/value tile it loads

struct PrefillParams {
    void *out;
    const void *q, *k, *v;
    const int32_t *tables, *ctx_lens, *query_start;
    uint32_t num_blocks;
    int32_t max_blocks, ctx_cap, num_q_heads, num_kv_heads, group;
    float scale_log2;
};

template <class E, int B, int W, int RT>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const PrefillParams p) {
    using M = Mfma<E>;
    constexpr int D = 128, TR = 16, SPB = B / TR, ROWB = D * 2, NS = kPrefillStages;
    static_assert(B % TR == 0, "block_size must be a multiple of 16");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int s = blockIdx.z, kvh = blockIdx.y;
    const int G = p.group;
    // per-sequence values, uniform (scalar registers): the buffer resources built from them
    // stay scalar, with no per-lane loop around the loads
    const int q0 = __builtin_amdgcn_readfirstlane(p.query_start[s]);
    const int nq = __builtin_amdgcn_readfirstlane(p.query_start[s + 1]) - q0;
    const int ctx = clamp_ctx(__builtin_amdgcn_readfirstlane(p.ctx_lens[s]), p.ctx_cap);
    const int rows = nq * G;
    const int row0 = (blockIdx.x * W + wave) * 16 * RT;  // the wave's RT row tiles start here
    if (nq <= 0 || nq > ctx || row0 >= rows) return;  // uniform over the wave

    // row n of each of the wave's row tiles: query token, head, position
    bool row_ok[RT];
    int tok[RT], head[RT], qpos[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = row0 + rt * 16 + n;
        row_ok[rt] = r < rows;
        tok[rt] = row_ok[rt] ? r / G : 0;
        head[rt] = kvh * G + (row_ok[rt] ? r % G : 0);
        qpos[rt] = ctx - nq + tok[rt];
    }
    const int last_tok = (min(row0 + 16 * RT - 1, rows - 1)) / G;
    // keys these rows need: [0, kend) (uniform: it sizes the loop and the buffer resources)
    const int kend = __builtin_amdgcn_readfirstlane(ctx - nq + last_tok + 1);
    const int ntile = (kend + TR - 1) / TR;

    u32x4 qv[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const char *qp = static_cast<const char *>(p.q) +
                         ((static_cast<int64_t>(q0 + tok[rt]) * p.num_q_heads + head[rt]) * D + g * 8) * 2;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qv[rt][kk] = row_ok[rt] ? *reinterpret_cast<const u32x4 *>(qp + kk * 64) : u32x4{0u, 0u, 0u, 0u};
    }

    TableEntry *trow = (TableEntry *)(p.tables + static_cast<int64_t>(s) * p.max_blocks);  // address-space cast
    const char *kc = static_cast<const char *>(p.k);
    const char *vc = static_cast<const char *>(p.v);
    const unsigned koff = n * ROWB + g * 16;      // + kk * 64: row n, chunk 4*kk + g
    const unsigned voff = g * 4 * ROWB + n * 16;  // + i * ROWB: row 4g + i, chunk n

    struct Stage {
        u32x4 k[4], v[4];
        int t;    // key tile (>= ntile: a stand-in)
        bool ok;  // table entry inside the pool
    };
    int ct = 0;  // next tile to issue; its table entry is looked up one tile ahead
    int cpb = trow[0];
    auto issue = [&](Stage &S) {
        S.t = ct;
        const int jt = min(ct, ntile - 1);
        S.ok = static_cast<uint32_t>(cpb) < p.num_blocks;
        const int64_t blk = S.ok ? cpb : 0;
        const int64_t tile = ((blk * p.num_kv_heads + kvh) * B + (jt % SPB) * TR) * ROWB;
        const int keys = ct < ntile && S.ok ? min(TR, kend - ct * TR) : 0;
        const auto kr_ = tile_rsrc(kc + tile, keys * ROWB), vr_ = tile_rsrc(vc + tile, keys * ROWB);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) S.k[kk] = kv_buffer_load<false>(kr_, koff + kk * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) S.v[i] = kv_buffer_load<false>(vr_, voff + i * ROWB);
        ++ct;
        cpb = trow[min(ct, ntile - 1) / SPB];
    };

    float m[RT], lsum[RT];
    f32x4 acc[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = -INFINITY;
        lsum[rt] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // one key tile against every row tile of the wave (the tile's loads serve RT * 16 rows)
    auto consume = [&](Stage &S) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) c = M::mma(S.k[kk], qv[rt][kk], c);
            float sc[4], mloc = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kpos = S.t * TR + 4 * g + i;  // a stand-in's keys all lie past kend
                const bool valid = S.ok && kpos <= qpos[rt] && kpos < kend;
                sc[i] = valid ? c[i] * p.scale_log2 : -INFINITY;
                mloc = fmaxf(mloc, sc[i]);
            }
            mloc = max_over_lane_groups(mloc);
            const float m_new = fmaxf(m[rt], mloc);
            const float m_ref = m_new == -INFINITY ? 0.f : m_new;
            if (__builtin_amdgcn_ballot_w64(m_new > m[rt]) != 0) {
                const float alpha = fast_exp2(m[rt] - m_ref);
                lsum[rt] *= alpha;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[rt][j] *= alpha;
            }
            const float e0 = fast_exp2(sc[0] - m_ref), e1 = fast_exp2(sc[1] - m_ref);
            const float e2 = fast_exp2(sc[2] - m_ref), e3 = fast_exp2(sc[3] - m_ref);
            const unsigned h01 = M::pack2(e0, e1), h23 = M::pack2(e2, e3);
            const unsigned r01 = M::pack2(e0 - M::value(h01 & 0xffffu), e1 - M::value(h01 >> 16));
            const unsigned r23 = M::pack2(e2 - M::value(h23 & 0xffffu), e3 - M::value(h23 >> 16));
            lsum[rt] = M::sum2(r23, M::sum2(r01, M::sum2(h23, M::sum2(h01, lsum[rt]))));
            const u32x2 ph = {h01, h23}, pr = {r01, r23};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = j >> 1;
                const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const u32x2 vt = {__builtin_amdgcn_perm(word(S.v[1], w), word(S.v[0], w), sel),
                                  __builtin_amdgcn_perm(word(S.v[3], w), word(S.v[2], w), sel)};
                acc[rt][j] = M::mma16(vt, pr, M::mma16(vt, ph, acc[rt][j]));
            }
            m[rt] = m_new;
        }
    };

    // ring of NS stages over the wave's key tiles; whole rounds, the end tested at a round's
    // start (straight-line rounds keep the wait counts exact; the last may consume stand-ins)
    Stage R[NS];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
        issue(R[i]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (;;) {
        if (R[0].t >= ntile) break;
#pragma unroll
        for (int rr = 0; rr < NS; ++rr) {
            issue(R[(rr + NS - 1) % NS]);
            consume(R[rr]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // each row's weight sum over the four lane groups; lane (n, g) holds d = 8 (4g + i) + j
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float l = lsum[rt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (row_ok[rt]) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const int64_t base = (static_cast<int64_t>(q0 + tok[rt]) * p.num_q_heads + head[rt]) * D;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) E::store(p.out, base + 8 * (4 * g + i) + j, acc[rt][j][i] * inv);
        }
    }
}

template <class E, int B>
int launch(const PrefillParams &p, int32_t max_query_len, int32_t num_seqs, hipStream_t stream) {
    const int64_t tiles = ceil_div(static_cast<int64_t>(max_query_len) * p.group, 16);
    const int64_t gx = ceil_div(tiles, kPrefillWaves * kPrefillRowTiles);
    if (gx > INT32_MAX) return fail(PKV_EINVAL, "pkv_paged_attention_prefill: max_query_len too large");
    hipLaunchKernelGGL((prefill_kernel<E, B, kPrefillWaves, kPrefillRowTiles>), dim3(static_cast<unsigned>(gx), p.num_kv_heads, num_seqs),
                       dim3(kPrefillWaves * 64), 0, stream, p);
    return hip_status(hipGetLastError(), "pkv_paged_attention_prefill launch");
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_paged_attention_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                                           int64_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *context_lens, const int32_t *query_start,
                                           int32_t max_query_len, int32_t max_context_len, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, float scale, int32_t dtype, uint32_t flags,
                                           hipStream_t stream) {
    const char *fn = "pkv_paged_attention_prefill";
    if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "%s: num_seqs %d outside [0, 65535]", fn, num_seqs);
    if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
    if (dtype != PKV_F16 && dtype != PKV_BF16)
        return fail(PKV_EUNSUPPORTED, "%s: dtype %d not built (f16, bf16)", fn, dtype);
    if (head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d not built (128)", fn, head_dim);
    if (block_size != 16 && block_size != 32)
        return fail(PKV_EUNSUPPORTED, "%s: block_size %d not built (16, 32)", fn, block_size);
    if (num_kv_heads <= 0 || num_kv_heads > 65535 || num_q_heads <= 0 || num_q_heads % num_kv_heads)
        return fail(PKV_EINVAL, "%s: num_q_heads %d must be a positive multiple of num_kv_heads %d", fn, num_q_heads,
                    num_kv_heads);
    if (max_query_len < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        num_blocks > INT32_MAX)
        return fail(PKV_EINVAL, "%s: bad sizes", fn);
    if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale is not finite", fn);
    if (flags) return fail(PKV_EINVAL, "%s: unknown flags %#x", fn, flags);
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return fail(PKV_EINVAL, "%s: NULL pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_EINVAL, "%s: out, q, k, v must be 16-byte aligned", fn);
    if (debug_validate()) {
        int rc = validate_attention(fn, context_lens, num_seqs, max_context_len, block_tables, max_blocks_per_seq,
                                    block_size, num_blocks, 0, stream);
        if (rc) return rc;
        rc = validate_query_start(fn, query_start, context_lens, num_seqs, max_query_len, stream);
        if (rc) return rc;
    }
    PrefillParams p{};
    p.out = out;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.tables = block_tables;
    p.ctx_lens = context_lens;
    p.query_start = query_start;
    p.num_blocks = static_cast<uint32_t>(num_blocks);
    p.max_blocks = max_blocks_per_seq;
    p.ctx_cap = static_cast<int32_t>(
        std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * block_size));
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_q_heads / num_kv_heads;
    p.scale_log2 = scale * 1.4426950408889634f;
    if (dtype == PKV_F16)
        return block_size == 32 ? launch<F16, 32>(p, max_query_len, num_seqs, stream)
                                : launch<F16, 16>(p, max_query_len, num_seqs, stream);
    return block_size == 32 ? launch<BF16, 32>(p, max_query_len, num_seqs, stream)
                            : launch<BF16, 16>(p, max_query_len, num_seqs, stream);
}
