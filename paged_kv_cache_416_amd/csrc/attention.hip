// Decode attention over a paged KV cache, one query token per sequence.
//
// "vLLM and PagedAttention" slide 9: attention is computed block by block;
// keys and values are fetched from non-contiguous blocks by address, through
// the block table (slide 10). The result is ordinary single-query scaled
// dot-product attention over the sequence's gathered context.
//
// Kernel design (gfx950, wave64):
//  * one workgroup = 4 waves per (sequence, query head[, partition]);
//  * the workgroup stages the block-table entries it needs in LDS, then each
//    wave walks its share of blocks; the (block, kv head) tile is B rows of
//    head_dim elements, contiguous in memory, and the wave reads it with
//    16-byte loads, consecutive lanes on consecutive 16 bytes (1 KiB per
//    instruction), K and V tiles of several blocks in flight at once;
//  * a row's dot product is split over LPR lanes and finished with a
//    cross-lane butterfly; softmax is online per wave (running max m, sum l,
//    rescaled accumulator), in base 2 with log2(e) folded into the scale;
//  * waves merge through LDS in a fixed order; no atomics, so results are
//    bit-reproducible and do not depend on where blocks live;
//  * rows past the context end are never loaded and are excluded by select,
//    never multiplied by a zero weight (0 * NaN = NaN);
//  * split mode: each partition writes (m, l, unnormalised accumulator) to
//    an fp32 workspace and a second kernel merges them:
//    M = max_p m_p, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// The contiguous-cache variant is the same template; only a tile's address differs.
#include <algorithm>
#include <cmath>

#include "common.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTableChunk = 256;  // block-table entries staged in LDS at a time

struct F32 {
    static constexpr int VEC = 4;
    static constexpr int ELT = 4;
    static __device__ inline void unpack(const u32x4 &r, float *f) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    static __device__ inline void store(void *out, int64_t i, float x) { static_cast<float *>(out)[i] = x; }
};

struct F16 {
    static constexpr int VEC = 8;
    static constexpr int ELT = 2;
    static __device__ inline void unpack(const u32x4 &r, float *f) {
        const f16x8 h = __builtin_bit_cast(f16x8, r);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(h[i]);
    }
    static __device__ inline void store(void *out, int64_t i, float x) {
        static_cast<_Float16 *>(out)[i] = static_cast<_Float16>(x);  // round to nearest even
    }
};

struct BF16 {
    static constexpr int VEC = 8;
    static constexpr int ELT = 2;
    static __device__ inline void unpack(const u32x4 &r, float *f) {
        const unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ inline void store(void *out, int64_t i, float x) {
        static_cast<__bf16 *>(out)[i] = static_cast<__bf16>(x);  // round to nearest even
    }
};

struct AttnParams {
    void *out;
    const void *q;
    const void *k;
    const void *v;
    const int32_t *tables;
    const int32_t *ctx_lens;
    float *ws;             // split workspace: acc [S*Hq*P][D], then m [S*Hq*P], then l [S*Hq*P]
    int64_t num_blocks;    // paged: pool size
    int64_t ws_rows;       // S * Hq * num_parts
    int32_t max_blocks;    // paged: table row stride
    int32_t lmax;          // contiguous: rows per (sequence, kv head)
    int32_t ctx_cap;       // lengths are clamped to [0, ctx_cap]
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;         // num_q_heads / num_kv_heads
    int32_t partition_size;  // 0 = single pass
    int32_t num_parts;       // workspace parts per (sequence, head)
    float scale_log2;        // scale * log2(e)
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

// Main kernel: grid = (parts, num_q_heads, num_seqs), block = 256.
// E: element type; D: head_dim; B: tokens per block (tile rows); PAGED: table lookup or contiguous slab.
template <class E, int D, int B, bool PAGED>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(const AttnParams p) {
    constexpr int VEC = E::VEC;         // elements per 16-byte load
    constexpr int LPR = D / VEC;        // lanes per tile row
    constexpr int RPI = 64 / LPR;       // tile rows per wave load instruction
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "head_dim does not map onto a wave");
    static_assert(B % RPI == 0, "block_size must be a multiple of rows per load");
    constexpr int NL = B / RPI;         // loads per lane per tile
    constexpr int U = NL >= 8 ? 1 : 8 / NL;  // tiles per wave iteration (K and V: 2*U*NL loads in flight)

    __shared__ int32_t s_tbl[PAGED ? kTableChunk : 1];
    __shared__ float s_m[kWaves], s_l[kWaves];
    __shared__ float s_acc[kWaves][D];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int part = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int kvh = h / p.group;
    const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
    int t0 = 0, t1 = ctx;
    if (p.partition_size > 0) {
        t0 = part * p.partition_size;
        t1 = min(ctx, t0 + p.partition_size);
    }
    const int64_t row_q = static_cast<int64_t>(s) * p.num_q_heads + h;
    if (t0 >= t1) {  // uniform over the workgroup
        if (p.partition_size == 0)
            for (int i = threadIdx.x; i < D; i += kThreads) E::store(p.out, row_q * D + i, 0.f);
        return;
    }

    const int r0 = lane / LPR, c = lane % LPR;
    float qf[VEC];
    {
        const char *qp = static_cast<const char *>(p.q) + (row_q * D + c * VEC) * E::ELT;
        E::unpack(*reinterpret_cast<const u32x4 *>(qp), qf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) qf[e] *= p.scale_log2;
    }

    const char *kb = static_cast<const char *>(p.k);
    const char *vb = static_cast<const char *>(p.v);
    const int jb = t0 / B, je = (t1 + B - 1) / B;
    float m_w = -INFINITY, l_w = 0.f;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

    for (int cb = jb; cb < je; cb += (PAGED ? kTableChunk : (1 << 30))) {
        const int n = PAGED ? min(kTableChunk, je - cb) : je - cb;
        if constexpr (PAGED) {
            __syncthreads();  // the previous chunk's entries are no longer read
            const int32_t *trow = p.tables + static_cast<int64_t>(s) * p.max_blocks + cb;
            for (int i = threadIdx.x; i < n; i += kThreads) s_tbl[i] = trow[i];
            __syncthreads();
        }
        for (int i0 = wave * U; i0 < n; i0 += kWaves * U) {
            u32x4 kr[U][NL], vr[U][NL];
            bool okb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = i0 + u;
                const int tok0 = (cb + j) * B;
                bool ok = j < n;
                int64_t tile;
                if constexpr (PAGED) {
                    const int pb = ok ? s_tbl[j] : 0;
                    ok = ok && pb >= 0 && pb < p.num_blocks;
                    tile = (static_cast<int64_t>(pb) * p.num_kv_heads + kvh) * (B * D);
                } else {
                    tile = ((static_cast<int64_t>(s) * p.num_kv_heads + kvh) * p.lmax + tok0) * D;
                }
                okb[u] = ok;
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    const int row = l * RPI + r0;
                    const int64_t off = (tile + static_cast<int64_t>(row) * D + c * VEC) * E::ELT;
                    if (ok && tok0 + row < t1) {
                        kr[u][l] = *reinterpret_cast<const u32x4 *>(kb + off);
                        vr[u][l] = *reinterpret_cast<const u32x4 *>(vb + off);
                    } else {
                        kr[u][l] = u32x4{0u, 0u, 0u, 0u};
                        vr[u][l] = u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }
            // logits (base 2) of this iteration's rows
            float sc[U][NL];
            float mloc = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int tok0 = (cb + i0 + u) * B;
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    float kf[VEC];
                    E::unpack(kr[u][l], kf);
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) d = fmaf(qf[e], kf[e], d);
#pragma unroll
                    for (int o = LPR / 2; o > 0; o >>= 1) d += __shfl_xor(d, o);
                    const bool ok = okb[u] && tok0 + l * RPI + r0 < t1;
                    sc[u][l] = ok ? d : -INFINITY;
                    mloc = fmaxf(mloc, sc[u][l]);
                }
            }
#pragma unroll
            for (int o = LPR; o < 64; o <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
            const float m_new = fmaxf(m_w, mloc);
            const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // only when every tile was rejected
            const float alpha = fast_exp2(m_w - m_ref);
            l_w *= alpha;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    const float pr = fast_exp2(sc[u][l] - m_ref);
                    l_w += pr;
                    float vf[VEC];
                    E::unpack(vr[u][l], vf);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[e] = fmaf(pr, vf[e], acc[e]);
                }
            }
            m_w = m_new;
        }
    }

    // sum over the wave's row groups: lanes with the same column chunk c
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
        l_w += __shfl_xor(l_w, o);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], o);
    }
    if (lane < LPR) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_acc[wave][c * VEC + e] = acc[e];
    }
    if (lane == 0) {
        s_m[wave] = m_w;
        s_l[wave] = l_w;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < D; i += kThreads) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w]);
        const float Mr = M == -INFINITY ? 0.f : M;
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(s_m[w] - Mr);
            L = fmaf(s_l[w], f, L);
            O = fmaf(s_acc[w][i], f, O);
        }
        if (p.partition_size > 0) {
            const int64_t wr = row_q * p.num_parts + part;
            p.ws[wr * D + i] = O;
            if (i == 0) {
                p.ws[p.ws_rows * D + wr] = M;
                p.ws[p.ws_rows * (D + 1) + wr] = L;
            }
        } else {
            E::store(p.out, row_q * D + i, L > 0.f ? O / L : 0.f);
        }
    }
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

template <class E, int D, int B, bool PAGED>
int launch(const AttnParams &p, int32_t num_seqs, int32_t grid_parts, hipStream_t stream) {
    hipLaunchKernelGGL((attn_decode_kernel<E, D, B, PAGED>), dim3(grid_parts, p.num_q_heads, num_seqs),
                       dim3(kThreads), 0, stream, p);
    int rc = hip_status(hipGetLastError(), "attention launch");
    if (rc || p.partition_size == 0) return rc;
    hipLaunchKernelGGL((attn_reduce_kernel<E, D>), dim3(p.num_q_heads, num_seqs), dim3(D), 0, stream, p);
    return hip_status(hipGetLastError(), "attention reduce launch");
}

template <class E, int D, bool PAGED>
int dispatch_block(const AttnParams &p, int32_t block_size, int32_t num_seqs, int32_t grid_parts,
                   hipStream_t stream) {
    switch (block_size) {
    case 8: return launch<E, D, 8, PAGED>(p, num_seqs, grid_parts, stream);
    case 16: return launch<E, D, 16, PAGED>(p, num_seqs, grid_parts, stream);
    case 32: return launch<E, D, 32, PAGED>(p, num_seqs, grid_parts, stream);
    default: return fail(PKV_EUNSUPPORTED, "block_size %d not built (8, 16, 32)", block_size);
    }
}

template <bool PAGED>
int dispatch(const AttnParams &p, int32_t dtype, int32_t head_dim, int32_t block_size, int32_t num_seqs,
             int32_t grid_parts, hipStream_t stream) {
#define PKV_HD(E)                                                                            \
    switch (head_dim) {                                                                      \
    case 64: return dispatch_block<E, 64, PAGED>(p, block_size, num_seqs, grid_parts, stream);   \
    case 128: return dispatch_block<E, 128, PAGED>(p, block_size, num_seqs, grid_parts, stream); \
    default: return fail(PKV_EUNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);     \
    }
    switch (dtype) {
    case PKV_F32: PKV_HD(F32)
    case PKV_F16: PKV_HD(F16)
    case PKV_BF16: PKV_HD(BF16)
    default: return fail(PKV_EINVAL, "bad dtype %d", dtype);
    }
#undef PKV_HD
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
    if (partition_size < 0) return fail(PKV_EINVAL, "%s: partition_size < 0", fn);
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k || !v || !context_lens) return fail(PKV_EINVAL, "%s: NULL pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(PKV_EINVAL, "%s: out, q, k, v must be 16-byte aligned", fn);
    if (partition_size > 0) {
        const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size);
        if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
            return fail(PKV_EINVAL, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn, need,
                        workspace ? workspace_bytes : 0);
    }
    return PKV_OK;
}

AttnParams make_params(void *out, const void *q, const void *k, const void *v, const int32_t *context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, float scale,
                       int32_t partition_size, int32_t max_context_len, int32_t ctx_cap, void *workspace) {
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
    return p;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t partition_size) {
    if (partition_size <= 0 || num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
    const int64_t parts = ceil_div(max_context_len, partition_size);
    return static_cast<size_t>(num_seqs) * num_q_heads * parts * (head_dim + 2) * sizeof(float);
}

extern "C" int pkv_paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                                          int64_t num_blocks, const int32_t *block_tables,
                                          int32_t max_blocks_per_seq, const int32_t *context_lens,
                                          int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                                          int32_t partition_size, void *workspace, size_t workspace_bytes,
                                          int32_t dtype, uint32_t flags, hipStream_t stream) {
    const char *fn = "pkv_paged_attention_decode";
    int rc = check_common(fn, out, q, k_cache, v_cache, context_lens, max_context_len, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, scale, partition_size, workspace, workspace_bytes, dtype);
    if (rc || num_seqs == 0) return rc;
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PKV_EUNSUPPORTED, "%s: block_size %d not built (8, 16, 32)", fn, block_size);
    if (partition_size % block_size)
        return fail(PKV_EINVAL, "%s: partition_size %d is not a multiple of block_size %d", fn, partition_size,
                    block_size);
    if (!block_tables || max_blocks_per_seq <= 0 || num_blocks <= 0)
        return fail(PKV_EINVAL, "%s: block_tables NULL or max_blocks_per_seq / num_blocks not positive", fn);
    (void)flags;
    const int64_t cap = std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * block_size);
    AttnParams p = make_params(out, q, k_cache, v_cache, context_lens, num_seqs, num_q_heads, num_kv_heads, scale,
                               partition_size, max_context_len, static_cast<int32_t>(cap), workspace);
    p.tables = block_tables;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    const int32_t grid_parts = p.partition_size ? static_cast<int32_t>(ceil_div(cap, p.partition_size)) : 1;
    return dispatch<true>(p, dtype, head_dim, block_size, num_seqs, grid_parts, stream);
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
    if (lmax <= 0) return fail(PKV_EINVAL, "%s: lmax must be positive", fn);
    // tile rows of the contiguous slab: 16 (any multiple of rows-per-load works)
    constexpr int32_t kTile = 16;
    if (partition_size % kTile) return fail(PKV_EINVAL, "%s: partition_size must be a multiple of 16", fn);
    (void)flags;
    const int32_t cap = std::min(max_context_len, lmax);
    AttnParams p = make_params(out, q, k, v, context_lens, num_seqs, num_q_heads, num_kv_heads, scale,
                               partition_size, max_context_len, cap, workspace);
    p.lmax = lmax;
    const int32_t grid_parts = p.partition_size ? static_cast<int32_t>(ceil_div(cap, p.partition_size)) : 1;
    return dispatch<false>(p, dtype, head_dim, kTile, num_seqs, grid_parts, stream);
}
