// Device-side pieces shared by the decode-attention kernels: element traits, launch
// parameters, lane helpers. Internal to libpkv (not part of the C ABI).
#pragma once

#include "common.h"

namespace pkv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));


__device__ inline float as_f(unsigned u) { return __uint_as_float(u); }

struct F32 {
    static constexpr int CODE = PKV_F32;
    static constexpr int VEC = 4;
    static constexpr int ELT = 4;
    static __device__ inline float dot(const u32x4 &q, const u32x4 &k, float a) {
        a = fmaf(as_f(q.x), as_f(k.x), a);
        a = fmaf(as_f(q.y), as_f(k.y), a);
        a = fmaf(as_f(q.z), as_f(k.z), a);
        return fmaf(as_f(q.w), as_f(k.w), a);
    }
    static __device__ inline void axpy(float p, const u32x4 &v, float *acc) {
        acc[0] = fmaf(p, as_f(v.x), acc[0]);
        acc[1] = fmaf(p, as_f(v.y), acc[1]);
        acc[2] = fmaf(p, as_f(v.z), acc[2]);
        acc[3] = fmaf(p, as_f(v.w), acc[3]);
    }
    static __device__ inline void store(void *out, int64_t i, float x) { static_cast<float *>(out)[i] = x; }
};

struct F16 {
    static constexpr int CODE = PKV_F16;
    static constexpr int VEC = 8;
    static constexpr int ELT = 2;
    static __device__ inline float dot(const u32x4 &q, const u32x4 &k, float a) {
        // products of binary16 values are exact in fp32; dot2 accumulates in fp32.
        // (Words are copied out of the vectors first: a bit_cast of a vector element
        // lvalue reads element 0 with this compiler.)
        const unsigned qw[4] = {q.x, q.y, q.z, q.w}, kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qw[i]), __builtin_bit_cast(f16x2, kw[i]), a, false);
        return a;
    }
    static __device__ inline void axpy(float p, const u32x4 &v, float *acc) {
        const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(p, static_cast<float>(h[i]), acc[i]);
    }
    static __device__ inline void store(void *out, int64_t i, float x) {
        static_cast<_Float16 *>(out)[i] = static_cast<_Float16>(x);  // round to nearest even
    }
};

struct BF16 {
    static constexpr int CODE = PKV_BF16;
    static constexpr int VEC = 8;
    static constexpr int ELT = 2;
    static __device__ inline float dot(const u32x4 &q, const u32x4 &k, float a) {
        const unsigned qw[4] = {q.x, q.y, q.z, q.w}, kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[i]), __builtin_bit_cast(bf16x2, kw[i]),
                                                a, false);
        return a;
    }
    static __device__ inline void axpy(float p, const u32x4 &v, float *acc) {
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(p, as_f(w[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(p, as_f(w[i] & 0xffff0000u), acc[2 * i + 1]);
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
    const int32_t *cached_lens;  // kLoadSplit: per sequence, tokens [0, n) are loaded through the caches
    // decode step with the cache write: sequence s's new key and value rows (its token at position
    // length - 1, [S][Hkv][D]) and their slot; null new_k for attention alone
    const void *new_k;
    const void *new_v;
    const int64_t *new_slots;
    int64_t num_slots;  // num_blocks * block_size: a slot at or past it is not written
    void *k_write;      // the caches again, writable (k and v above), for the new rows
    void *v_write;
    float *ws;             // split workspace: acc [S*Hq*P][D], then m [S*Hq*P], then l [S*Hq*P]
    int64_t ws_rows;       // S * Hq * num_parts
    uint32_t num_blocks;   // paged: pool size (< 2^31)
    int32_t max_blocks;    // paged: table row stride
    int32_t lmax;          // contiguous: rows per (sequence, kv head)
    int32_t ctx_cap;       // lengths are clamped to [0, ctx_cap]
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;         // num_q_heads / num_kv_heads
    int32_t partition_size;  // 0 = single pass, > 0 = fixed partitions, PKV_PARTITION_BALANCED
    int32_t num_parts;       // workspace parts per (sequence, head)
    float scale_log2;        // scale * log2(e)
    int32_t num_seqs;
    int32_t head_dim;
    size_t ws_bytes;
    int32_t balanced_wgs;    // balanced schedule: workgroups sharing the batch's tiles
    int32_t tile_rows;       // balanced schedule: rows (tokens) per tile
    int32_t rows_per_seq;    // balanced schedule: work rows per sequence (query heads, or kv heads)
    int32_t heads_per_row;   // balanced schedule: query heads one work row serves
    int32_t head_major;      // balanced schedule: rows ordered head-major (1) or sequence-major (0)
};

// Where a workgroup's merged result for one work row goes: acc == nullptr means the final,
// normalised output in the element type; otherwise the unnormalised accumulator, the running
// max m and the sum l of each head (head j at acc + j*acc_stride, m + j*ml_stride, l + ...).
struct Sink {
    float *acc;
    float *m;
    float *l;
    int64_t acc_stride;
    int64_t ml_stride;
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

// ---------------------------------------------------------------- balanced schedule
// The work rows of the batch, each cut into tiles of tile_rows tokens, form one list of T tiles,
// sequence-major (row = s * rows_per_seq + h) or head-major (row = h * num_seqs + s). Workgroup
// g takes the share v = virtual(g) of it, tiles [b(v), b(v+1)), b(v) = floor(v*T/W). Workgroups
// are dealt to the 8 XCDs round-robin, so virtual() gives each XCD a contiguous run of shares:
// with head-major rows an XCD then serves few kv heads, and a block that many sequences share
// stays in that XCD's L2. A row one workgroup holds whole is written to the output; a row cut
// between workgroups leaves one partial result per share in the workspace (slot 2v for the
// share's first row, 2v+1 for its last), merged in share order by attn_reduce_balanced_kernel.
constexpr int kBalancedMaxSeqs = 4096;
constexpr int kBalancedWgsPerCu = 2;
constexpr int kXcds = 8;

// Fixed partitions of the grouped-query kernel on the persistent schedule (attention_gqa.hip):
// one workgroup of kGqaPartsWaves waves per CU, each wave an equal share of the tile list.
// Its workspace: the partition rows every fixed-partition launch uses (acc [rows][D], then m
// [rows], then l [rows], rows = num_seqs * num_q_heads * num_parts), padded to 16 bytes; then
// one slot per (wave, query head of the group) for a piece of a partition cut by a share
// boundary (acc [slots][D], m [slots], l [slots]); then the prefix sums C (kBalancedMaxSeqs + 1);
// then one flag per work row (kv head, sequence): merged by the attention kernel.
constexpr int kGqaPartsWaves = 8;
constexpr int kGqaMaxGroup = 16;

__host__ __device__ inline int64_t parts_slot_offset(int64_t ws_rows, int64_t head_dim) {
    return (ws_rows * (head_dim + 2) + 3) / 4 * 4;
}
__host__ __device__ inline int64_t parts_slot_count(int64_t wgs, int64_t group) { return wgs * kGqaPartsWaves * group; }
__host__ __device__ inline int64_t parts_prefix_offset(int64_t ws_rows, int64_t head_dim, int64_t slots) {
    return parts_slot_offset(ws_rows, head_dim) + slots * (head_dim + 2);
}
__host__ __device__ inline size_t parts_workspace_bytes(int64_t ws_rows, int64_t head_dim, int64_t slots,
                                                        int64_t work_rows) {
    return static_cast<size_t>(parts_prefix_offset(ws_rows, head_dim, slots) + kBalancedMaxSeqs + 1 + work_rows) * 4;
}

// floor(v T / nwg) in double precision (a 64-bit integer division is a long instruction sequence
// on the GPU). Exact while v T < 2^53 (v <= nwg < 2^20, T < 2^31): a quotient that is an integer is
// represented exactly, and any other lies at least 1 / nwg from the integers, more than the
// rounding error q 2^-53 < 2^-22.
__device__ inline int64_t balanced_begin(int64_t v, int64_t T, int64_t nwg) {
    return static_cast<int64_t>(static_cast<double>(v * T) / static_cast<double>(nwg));
}

// The share holding tile x (0 <= x < T): floor(((x + 1) nwg - 1) / T), taken in double precision
// (a 64-bit integer division is a long instruction sequence on the GPU). Exact while T nwg < 2^53:
// the numerator converts exactly, the quotient is below nwg, so the rounded quotient is within
// nwg 2^-53 of the true one, while a true quotient below an integer k is at most k - 1/T.
__device__ inline int64_t balanced_owner(int64_t x, int64_t T, int64_t nwg) {
    return static_cast<int64_t>(static_cast<double>((x + 1) * nwg - 1) / static_cast<double>(T));
}

__device__ inline int64_t balanced_virtual(int64_t g, int64_t nwg) {
    return nwg % kXcds == 0 ? (g % kXcds) * (nwg / kXcds) + g / kXcds : g;
}

// Where the prefix sums C live in the workspace: after the 2 * balanced_wgs result slots.
__device__ inline uint32_t *balanced_prefix_out(const AttnParams &p) {
    return reinterpret_cast<uint32_t *>(p.ws + 2 * static_cast<int64_t>(p.balanced_wgs) * p.heads_per_row *
                                                   (p.head_dim + 2));
}

// One record per share, after C: the (sequence, head) of the cut row whose last tile the share
// holds (the merge pass merges that row), or -1.
__device__ inline int32_t *balanced_records(const AttnParams &p) {
    return reinterpret_cast<int32_t *>(balanced_prefix_out(p) + kBalancedMaxSeqs + 1);
}

// C[s] = tiles per row of the sequences before s, for s = 0 .. S (LDS, all threads of the
// block); lengths clamped as everywhere else. Ends with a barrier (except workgroup 0's copy
// of C to `out` in the workspace, which the merge pass reads after this kernel).
template <int NT>
__device__ inline void balanced_prefix(const AttnParams &p, uint32_t *C, uint32_t *part, uint32_t *out) {
    const int t = threadIdx.x, S = p.num_seqs, TR = p.tile_rows;
    const int per = (S + NT - 1) / NT, s0 = t * per;
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i)
        if (s0 + i < S) sum += (clamp_ctx(p.ctx_lens[s0 + i], p.ctx_cap) + TR - 1) / TR;
    part[t] = sum;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
        const uint32_t v = t >= o ? part[t - o] : 0u;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint32_t run = t > 0 ? part[t - 1] : 0u;
    for (int i = 0; i < per; ++i)
        if (s0 + i < S) {
            C[s0 + i] = run;
            run += (clamp_ctx(p.ctx_lens[s0 + i], p.ctx_cap) + TR - 1) / TR;
        }
    if (t == NT - 1) C[S] = part[NT - 1];
    __syncthreads();
    // workgroup 0 leaves C in the workspace, after the slots, for the merge pass
    if (blockIdx.x == 0)
        for (int i = t; i <= S; i += NT) out[i] = C[i];
}

// Decode step with the cache write: 16-byte chunk `chunk` of sequence s's new key and value rows
// for kv head kvh goes to the token's slot (slide 11: a new token goes into the free slot of its
// sequence's last block). Called only where new_row_position(p, s) >= 0 (a slot inside the pool).
// Nothing in the launch reads what this writes: attention takes that row from new_k/new_v.
template <int B, int ROWB>
__device__ inline void store_new_row(const AttnParams &p, int s, int kvh, int chunk, const u32x4 &k, const u32x4 &v) {
    const int64_t slot = p.new_slots[s];
    const int64_t blk = slot / B, off = slot - blk * B;
    const int64_t dst = ((blk * p.num_kv_heads + kvh) * B + off) * ROWB + chunk * 16;
    *reinterpret_cast<u32x4 *>(static_cast<char *>(p.k_write) + dst) = k;
    *reinterpret_cast<u32x4 *>(static_cast<char *>(p.v_write) + dst) = v;
}

// Decode step with the cache write: the position of sequence s's new token if this launch writes
// it (a slot inside the pool, a non-empty sequence), else -1 (attention alone, or a row the cache
// already holds: a negative slot, which an empty sequence must have). Uniform.
__device__ inline int new_row_position(const AttnParams &p, int s) {
    if (!p.new_k) return -1;
    const int64_t slot = p.new_slots[s];
    const int ctx = clamp_ctx(p.ctx_lens[s], p.ctx_cap);
    return __builtin_amdgcn_readfirstlane(slot >= 0 && slot < p.num_slots && ctx > 0 ? ctx - 1 : -1);
}

// Outputs of sequences with no tokens are zeros; the workgroups share them out.
template <class E, int D, int NT>
__device__ inline void balanced_zero_empty(const AttnParams &p, const uint32_t *C) {
    for (int s = blockIdx.x; s < p.num_seqs; s += gridDim.x)
        if (C[s + 1] == C[s])
            for (int i = threadIdx.x; i < p.num_q_heads * D; i += NT)
                E::store(p.out, static_cast<int64_t>(s) * p.num_q_heads * D + i, 0.f);
}

// Row of list position x (0 <= x < T): its sequence s, head h and first tile's position row0.
template <bool HEAD_MAJOR>
__device__ inline void balanced_locate(const uint32_t *C, int S, int64_t R, int64_t x, int &s, int &h,
                                       int64_t &row0) {
    const int64_t Ctot = C[S];
    int64_t rem = x;
    if constexpr (HEAD_MAJOR) {
        h = static_cast<int>(x / Ctot);
        rem = x - h * Ctot;
    }
    const int64_t scale = HEAD_MAJOR ? 1 : R;
    int lo = 0, hi = S;  // largest s with scale*C[s] <= rem: it has tiles (scale*C[s+1] > rem)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (scale * C[mid] <= rem) lo = mid; else hi = mid;
    }
    s = lo;
    if constexpr (HEAD_MAJOR) {
        row0 = h * Ctot + C[s];
    } else {
        const int64_t n = C[s + 1] - C[s];
        h = static_cast<int>((x - R * C[s]) / n);
        row0 = R * C[s] + h * n;
    }
}

// Walk this workgroup's share: body(s, h, tile_begin, tile_end, sink) per row segment, in order.
// Uniform over the workgroup.
template <int D, bool HEAD_MAJOR, class Body>
__device__ inline void balanced_walk(const AttnParams &p, const uint32_t *C, Body &&body) {
    const int64_t R = p.rows_per_seq, nwg = p.balanced_wgs;
    const int64_t T = R * C[p.num_seqs];
    const int64_t v = balanced_virtual(blockIdx.x, nwg);
    int32_t *rec = balanced_records(p) + 2 * v;
    if (threadIdx.x == 0) rec[0] = rec[1] = -1;
    if (T == 0) return;
    int64_t pos = balanced_begin(v, T, nwg);
    const int64_t end = balanced_begin(v + 1, T, nwg);
    const int64_t slot_floats = static_cast<int64_t>(p.heads_per_row) * (D + 2);
    bool first = true;
    while (pos < end) {
        int s, h;
        int64_t row0;
        balanced_locate<HEAD_MAJOR>(C, p.num_seqs, R, pos, s, h, row0);
        const int64_t n = C[s + 1] - C[s];
        const int ta = static_cast<int>(pos - row0);
        const int tb = static_cast<int>(end - row0 < n ? end - row0 : n);
        Sink sink{nullptr, nullptr, nullptr, 0, 0};
        if (ta != 0 || tb != n) {
            float *slot = p.ws + (2 * v + (first ? 0 : 1)) * slot_floats;
            sink = Sink{slot, slot + p.heads_per_row * D, slot + p.heads_per_row * (D + 1), D, 1};
        }
        if (first && ta != 0 && tb == n && threadIdx.x == 0) {  // this share ends a cut row: merge it
            rec[0] = s;
            rec[1] = h;
        }
        body(s, h, ta, tb, sink);
        first = false;
        pos = row0 + tb;
    }
}

// DPP lane moves within a row of 16 lanes.
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within each 16 lanes

template <int CTRL>
__device__ inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of N consecutive lanes (N = 8, 16, 32 or 64); every lane of
// the group gets the same value (each step adds a lane's value to its partner's, and
// floating-point addition is commutative).
template <int N>
__device__ inline float group_sum(float x) {
    static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    x += dpp<kRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

__device__ inline u32x4 nt_load(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// A buffer resource over the bytes [base, base + bytes) (raw, stride 0): a load whose offset
// lies at or past the end returns zeros, so the hardware range check masks rows past a
// sequence's end, and a zero-byte resource makes a tile read as zeros.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, uint32_t bytes) {
    constexpr int kRawBufferConfig = 0x00020000;  // dword 3 of a gfx9 raw buffer descriptor
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, static_cast<int>(bytes), kRawBufferConfig);
}

// How a kernel loads K/V: non-temporal, for blocks read once per call; through the caches, for
// blocks several sequences of the batch read (a shared prefix), whose re-reads then hit the L2
// or the last-level cache instead of HBM; or split per sequence: its first cached_lens[s]
// tokens through the caches (the blocks it shares), the rest non-temporal. The policy changes
// no arithmetic.
enum LoadPolicy { kLoadStream = 0, kLoadCached = 1, kLoadSplit = 2 };

// K/V loads. NT: non-temporal; otherwise through the caches.
template <bool NT>
__device__ inline u32x4 kv_load(const char *p) {
    if constexpr (NT) return nt_load(p);
    else return *reinterpret_cast<const u32x4 *>(p);
}

template <bool NT>
__device__ inline u32x4 kv_buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    constexpr int kPolicy = NT ? 2 : 0;  // cache-policy bit nt
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kPolicy);
}

// Compile-time shape of the tile walk for element type E, head_dim D, block_size B.

// MFMA grouped-query kernel (attention_gqa.hip). gqa_mfma_supported tells whether a shape has
// an MFMA build; launch_gqa_mfma enqueues it (and the reduce pass in split mode).
bool gqa_mfma_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group);
int launch_gqa_mfma(const AttnParams &p, int32_t dtype, int32_t block_size, bool paged, int load_policy,
                    int32_t num_seqs, int32_t grid_parts, hipStream_t stream);
// The partition merge (attention.hip), shared by both kernels.
int launch_reduce(const AttnParams &p, int32_t dtype, int32_t head_dim, int32_t num_seqs, hipStream_t stream);
// The balanced schedule's merge of cut rows (attention.hip).
int launch_reduce_balanced(const AttnParams &p, int32_t dtype, int32_t head_dim, hipStream_t stream);
// Compute units of the current device (cached), or -1.
int device_compute_units();
// Sets p.balanced_wgs (wgs_per_cu workgroups per compute unit, at most kBalancedWgsPerCu) and
// checks the balanced schedule's limits and workspace (p.tile_rows and p.heads_per_row set by
// the caller).
int balanced_check(AttnParams &p, int wgs_per_cu = kBalancedWgsPerCu);

}  // namespace pkv
