// Prefill (chunked) attention over the paged cache on the matrix cores: each sequence's last n_s
// tokens are queries, and query i (at position p = ctx - n_s + i) attends causally to the keys at
// positions 0 .. p, earlier chunks and shared prefix blocks included ("vLLM and PagedAttention"
// slide 3: the prompt is processed in parallel; slides 9 and 10: keys and values are fetched
// block by block through the block table).
//
// Matrix rows are (query token, query head) pairs of one kv head: row r of a sequence and kv
// head is token r / G, head kvh * G + r % G. A workgroup owns W * RT * 16 consecutive rows (each
// wave RT tiles of 16) and walks the keys up to its last row's position in steps of 32:
//  * the step's keys and values (16 KiB, two 16-key tiles) are read once per workgroup, whole
//    rows per load, through the block table, and written to a double-buffered LDS ring (rows
//    padded to 288 bytes: each row starts eight banks after the one before, which leaves both
//    operand reads below free of bank conflicts); one barrier per step;
//  * logits: S^T[key][row] = K[key][:] . Q^T[:][row] as 4 v_mfma_f32_16x16x32 per 16-key tile;
//  * weighted sum: O^T[d][row] = V^T[d][key] . P^T[key][row] as 8 v_mfma_f32_16x16x32 per
//    16-bit part of the weights, the k slots 8g .. 8g+7 of lane group g taking keys 4g .. 4g+3 of
//    the first tile and of the second, which is where the logits put them;
//  * the causal mask is a per-lane compare of the key's position with row n's position.
// Rows are independent: a wave writes its rows and ends; the workgroups that need the most keys
// (the last rows of each sequence) are dispatched first.
#include "mfma.h"

namespace pkv {
namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowTiles = 2;  // 16-row tiles per wave
constexpr int kStepKeys = 32;        // keys per step (two 16-key tiles)
constexpr int kLdsRow = 288;         // bytes per staged row: 256 + 32 of padding
constexpr float kMaxSlack = 8.f;     // log2 units the softmax reference may lag the running maximum

struct PrefillParams {
    void *out;
    const void *q, *k, *v;
    const int32_t *tables, *ctx_lens, *query_start;
    uint32_t num_blocks;
    int32_t num_tokens, max_blocks, ctx_cap, num_q_heads, num_kv_heads, group;
    float scale_log2;
};


// POS: the scale is positive, so the maximum of the scaled logits is the scale times the
// maximum of the raw ones, and each weight's exponent is one fma of its raw logit.
template <class E, int B, int W, int RT, bool POS>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const PrefillParams p) {
    using M = Mfma<E>;
    constexpr int D = 128, TR = 16, ROWB = D * 2, NT = W * 64, CPT = 2 * TR * 16 / NT;
    static_assert(B % TR == 0 && CPT >= 1 && 2 * TR * 16 % NT == 0, "shape");
    __shared__ __attribute__((aligned(16))) char lds[2][2][kStepKeys][kLdsRow];  // [buffer][K, V][key][byte]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int kvh = blockIdx.x, s = blockIdx.y;
    const int G = p.group;
    // per-sequence values, uniform (scalar registers): the buffer resources built from them
    // stay scalar, with no per-lane loop around the loads
    const int q0 = __builtin_amdgcn_readfirstlane(p.query_start[s]);
    const int nq = __builtin_amdgcn_readfirstlane(p.query_start[s + 1]) - q0;
    const int ctx = clamp_ctx(__builtin_amdgcn_readfirstlane(p.ctx_lens[s]), p.ctx_cap);
    const int rows = nq * G;
    const int wg_row0 = (gridDim.z - 1 - blockIdx.z) * W * RT * 16;
    // uniform over the workgroup; a sequence whose rows are not all inside q and out is skipped
    if (nq <= 0 || nq > ctx || q0 < 0 || q0 > p.num_tokens - nq || wg_row0 >= rows) return;
    const int row0 = wg_row0 + wave * RT * 16;  // a wave past the last row still loads and waits

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
    // the position of each row tile's first row: no row of the tile sees fewer keys
    int qmin[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) qmin[rt] = ctx - nq + (row0 + rt * 16) / G;
    // keys the workgroup needs: [0, kend); keys this wave's rows need: [0, kend_w)
    const int kend = __builtin_amdgcn_readfirstlane(ctx - nq + min(wg_row0 + W * RT * 16 - 1, rows - 1) / G + 1);
    const int kend_w = row0 < rows ? ctx - nq + min(row0 + RT * 16 - 1, rows - 1) / G + 1 : 0;
    const int nstep = (kend + kStepKeys - 1) / kStepKeys;

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

    // global loads of one step: thread chunk c = tid + k * NT is row c / 16 (its 16-key tile u =
    // row / 16, uniform over a wave), 16-byte column c % 16
    struct Stage {
        u32x4 k[CPT], v[CPT];
        int t;        // step (>= nstep: a stand-in)
        bool ok[2];   // table entries inside the pool
    };
    int ct = 0;  // next step to issue; its table entries are looked up one step ahead
    int cp[2] = {trow[0], trow[min(TR, kend - 1) / B]};
    auto issue = [&](Stage &S) {
        S.t = ct;
        int64_t tile[2];
        int bytes[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int kb = ct * kStepKeys + u * TR;
            S.ok[u] = static_cast<uint32_t>(cp[u]) < p.num_blocks;
            const int64_t blk = S.ok[u] ? cp[u] : 0;
            tile[u] = ((blk * p.num_kv_heads + kvh) * B + kb % B) * ROWB;
            // uniform, but the clamp is done with a vector instruction: readfirstlane keeps the
            // descriptor scalar
            bytes[u] = __builtin_amdgcn_readfirstlane((ct < nstep && S.ok[u] ? max(0, min(TR, kend - kb)) : 0) * ROWB);
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            // the chunk's 16-key tile: known at compile time up to 256 threads, else the wave's
            // half of the workgroup; the scalar inputs are selected, not the descriptors (a
            // select of descriptors is done per lane and would loop over the lanes at each load)
            const int u = NT <= 256 ? (k * NT) >> 8 : wave >> 2;
            const int c = tid + k * NT;
            const unsigned off = ((c >> 4) & 15) * ROWB + (c & 15) * 16;
            const int64_t tu = u ? tile[1] : tile[0];
            const int bu = u ? bytes[1] : bytes[0];
            S.k[k] = kv_buffer_load<false>(tile_rsrc(kc + tu, bu), off);
            S.v[k] = kv_buffer_load<false>(tile_rsrc(vc + tu, bu), off);
        }
        ++ct;
#pragma unroll
        for (int u = 0; u < 2; ++u) cp[u] = trow[min(ct * kStepKeys + u * TR, kend - 1) / B];
    };

    float m[RT];
    const unsigned one2 = M::pack2(1.f, 1.f);
    const u32x4 kOnes = {one2, one2, one2, one2};
    f32x4 lsum[RT];  // row n's weight sum in every element of lane (n, g): the all-ones product
    f32x4 acc[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = -INFINITY;
        lsum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // the staged step in buffer b against every row tile of the wave
    auto consume = [&](int b, int t, const bool ok[2]) {
        // The two matrix-core sections (the logits; the weighted sums with the second tile's
        // weights) run at raised wave priority: the other wave of the SIMD, from another
        // workgroup, then fills the issue slots around them instead of delaying them.
        __builtin_amdgcn_s_setprio(1);
        f32x4 c[RT][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            u32x4 kf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kf[kk] = *reinterpret_cast<const u32x4 *>(&lds[b][0][u * TR + n][(4 * kk + g) * 16]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                c[rt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) c[rt][u] = M::mma(kf[kk], qv[rt][kk], c[rt][u]);
            }
        }
        // V^T operand of weighted-sum MFMA j (d = 16 j + n): k slots 8g .. 8g+3 are keys 4g .. 4g+3
        // of the first 16-key tile and 8g+4 .. 8g+7 the same keys of the second, one transposed
        // LDS read each (lane (n, g) addresses row 4g + n / 4, columns 16 j + 4 (n % 4) .. + 3)
        u32x4 vt[8];
        {
            const char *vb = &lds[b][1][4 * g + (n >> 2)][(n & 3) * 8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const u32x2 a = lds_read_tr16(vb + j * 32), c2 = lds_read_tr16(vb + TR * kLdsRow + j * 32);
                vt[j] = u32x4{a.x, a.y, c2.x, c2.y};
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // The row tiles' softmax runs phase by phase over all of them, with one branch per phase
        // at most, so the tiles' independent chains share basic blocks and interleave.
        float sc[RT][2][4], mloc[RT];
        // a step wholly before a row tile's first row (and inside the pool) needs no mask; the
        // tiles' first rows grow with the tile index, so the first tile's test covers them all
        if ((t + 1) * kStepKeys - 1 <= qmin[0] && ok[0] && ok[1]) {  // uniform
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                mloc[rt] = -INFINITY;
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sc[rt][u][i] = POS ? c[rt][u][i] : c[rt][u][i] * p.scale_log2;
                        mloc[rt] = fmaxf(mloc[rt], sc[rt][u][i]);
                    }
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                mloc[rt] = -INFINITY;
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kpos = t * kStepKeys + u * TR + 4 * g + i;  // qpos < kend: kend is implied
                        const float x = POS ? c[rt][u][i] : c[rt][u][i] * p.scale_log2;
                        sc[rt][u][i] = ok[u] && kpos <= qpos[rt] ? x : -INFINITY;
                        mloc[rt] = fmaxf(mloc[rt], sc[rt][u][i]);
                    }
            }
        }
        // m[rt] is the reference the weights are taken against, exp2(s - m). It moves to the
        // running maximum only when some row's maximum passes it by more than kMaxSlack, so the
        // rescale is rare; the weights stay below 2^kMaxSlack, and the quotient acc / l does not
        // depend on the reference.
        bool grow = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) grow = grow || (POS ? mloc[rt] * p.scale_log2 : mloc[rt]) > m[rt] + kMaxSlack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            float m_new[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float mx = max_over_lane_groups(mloc[rt]);
                m_new[rt] = fmaxf(m[rt], POS ? mx * p.scale_log2 : mx);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float ref = m_new[rt] == -INFINITY ? 0.f : m_new[rt];
                const float alpha = fast_exp2(m[rt] - ref);
#pragma unroll
                for (int i = 0; i < 4; ++i) lsum[rt][i] *= alpha;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[rt][j] *= alpha;
                m[rt] = m_new[rt];
            }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float m_ref = m[rt] == -INFINITY ? 0.f : m[rt];
            unsigned h[4], r[4];  // weights of keys (u, 2w), (u, 2w + 1) in word 2u + w
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const float a0 = sc[rt][u][2 * w], a1 = sc[rt][u][2 * w + 1];
                    const float e0 = fast_exp2(POS ? fmaf(a0, p.scale_log2, -m_ref) : a0 - m_ref);
                    const float e1 = fast_exp2(POS ? fmaf(a1, p.scale_log2, -m_ref) : a1 - m_ref);
                    const unsigned hw = M::pack2(e0, e1);
                    h[2 * u + w] = hw;
                    r[2 * u + w] = M::pack2(e0 - M::lo(hw), e1 - M::hi(hw));
                }
            const u32x4 ph = {h[0], h[1], h[2], h[3]}, pr = {r[0], r[1], r[2], r[3]};
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[rt][j] = M::mma(vt[j], pr, M::mma(vt[j], ph, acc[rt][j]));
            // the weight sums on the matrix cores: an all-ones operand in place of V^T gives
            // every row of the product the column sum of P^T, the same fp32 accumulation
            lsum[rt] = M::mma(kOnes, pr, M::mma(kOnes, ph, lsum[rt]));
        }
        // the first row tile's weighted sum beside the second's weights: its 18 MFMAs among the
        // second tile's vector instructions
        __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
#pragma unroll
        for (int i = 0; i < 18; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // one step: stage the loaded rows in LDS, reuse the registers for the step two ahead, wait
    // for every wave's rows, compute (a wave whose rows need none of these keys skips it)
    auto step = [&](Stage &S, int b) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int c = tid + k * NT;
            *reinterpret_cast<u32x4 *>(&lds[b][0][c >> 4][(c & 15) * 16]) = S.k[k];
            *reinterpret_cast<u32x4 *>(&lds[b][1][c >> 4][(c & 15) * 16]) = S.v[k];
        }
        const int t = S.t;
        const bool ok[2] = {S.ok[0], S.ok[1]};
        issue(S);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t * kStepKeys < kend_w) consume(b, t, ok);
        __builtin_amdgcn_sched_barrier(0);
    };

    // two register stages in a ring; whole rounds, the end tested at a round's start (straight-
    // line rounds keep the wait counts exact; the last may be a stand-in step). Every wave runs
    // the same number of steps, so the barriers match.
    Stage R[2];
    __builtin_amdgcn_sched_barrier(0);
    issue(R[0]);
    __builtin_amdgcn_sched_barrier(0);
    issue(R[1]);
    __builtin_amdgcn_sched_barrier(0);
    for (;;) {
        if (R[0].t >= nstep) break;
        step(R[0], 0);
        step(R[1], 1);
    }

    // lane (n, g) holds row n's weight sum and d = 16 j + 4g + i of its output: four adjacent
    // outputs per j, rounded to nearest even and stored as one 8-byte word
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float l = lsum[rt][0];
        if (row_ok[rt]) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
            char *base = static_cast<char *>(p.out) +
                         (static_cast<int64_t>(q0 + tok[rt]) * p.num_q_heads + head[rt]) * D * 2;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const f32x4 a = acc[rt][j];
                *reinterpret_cast<u32x2 *>(base + (16 * j + 4 * g) * 2) =
                    u32x2{M::pack2(a[0] * inv, a[1] * inv), M::pack2(a[2] * inv, a[3] * inv)};
            }
        }
    }
}

template <class E, int B>
int launch(const PrefillParams &p, int32_t max_query_len, int32_t num_seqs, hipStream_t stream) {
    const int64_t tiles = ceil_div(static_cast<int64_t>(max_query_len) * p.group, 16);
    const int64_t gz = ceil_div(tiles, kPrefillWaves * kPrefillRowTiles);
    if (gz > 65535) return fail(PKV_EINVAL, "pkv_paged_attention_prefill: max_query_len too large");
    // Grid (kv heads, sequences, row blocks), the row blocks last and in reverse: workgroups are
    // dispatched in linear order, so every (kv head, sequence) pair's last rows, which need the
    // most keys, go first, and the light first rows of all pairs fill in at the end (longest
    // first). The kv head fastest deals each kv head to one XCD, whose L2 then holds its keys.
    const dim3 grid(p.num_kv_heads, num_seqs, static_cast<unsigned>(gz));
    if (p.scale_log2 > 0.f)
        hipLaunchKernelGGL((prefill_kernel<E, B, kPrefillWaves, kPrefillRowTiles, true>), grid, dim3(kPrefillWaves * 64),
                           0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<E, B, kPrefillWaves, kPrefillRowTiles, false>), grid, dim3(kPrefillWaves * 64),
                           0, stream, p);
    return hip_status(hipGetLastError(), "pkv_paged_attention_prefill launch");
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_paged_attention_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                                           int64_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *context_lens, const int32_t *query_start,
                                           int32_t num_tokens, int32_t max_query_len, int32_t max_context_len,
                                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                                           uint32_t flags, hipStream_t stream) {
    const char *fn = "pkv_paged_attention_prefill";
    if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "%s: num_seqs %d outside [0, 65535]", fn, num_seqs);
    if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens %d < 0", fn, num_tokens);
    if (num_seqs == 0 || max_query_len == 0 || num_tokens == 0) return PKV_OK;
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
        rc = validate_query_start(fn, query_start, context_lens, num_seqs, num_tokens, max_query_len, stream);
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
    p.num_tokens = num_tokens;
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
