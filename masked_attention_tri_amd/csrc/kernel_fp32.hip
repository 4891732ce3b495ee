// fp32 forward on the matrix core (v_mfma_f32_32x32x2_f32), for fp32 inputs
// (head dimension D <= 32, a multiple of 4: the triangle_attention page's
// envelope for fp32, Notes item 3) with no mask, kv_lengths, a dense key
// mask, a BlockMask whose query blocks are 32 or 64 rows or whole 128-row
// tiles and whose key blocks are 16 keys or whole 32-key tiles, or packed
// sequences (the Transformer Engine page's layouts, no mask or causal);
// other block sizes stay on the generic kernel.
//
// A workgroup of 4 waves takes 128 query rows of one (b, n, h), wave w rows
// 32w .. 32w+31, lane l the row 32w + l%32.  Keys go in tiles of 32, staged
// in LDS by the whole workgroup.  Both products are 16 k-steps of the 32 x 32
// x 2 MFMA, each k-step pairing two values of the summed index:
//   S^T = K . Q^T   step s pairs d = s and d = s + 16: lane l gives K[l%32][s +
//                   16 (l/32)] (A, from LDS) and Q[row][s + 16 (l/32)] (B,
//                   held in 16 registers for the whole key loop);
//   O^T = V^T . P^T step r pairs keys 8(r/4) + r%4 and that key + 4, which is
//                   where the accumulator of S^T puts them: register r of
//                   lane l holds key 8(r/4) + 4(l/32) + r%4 of row l%32, so
//                   the B operand of step r is the lane's own p[r], and the A
//                   operand is V[that key][l%32] from LDS.
// The softmax is the max-shifted online one in fp32 with expf: per tile the
// row max is raised and O and the sum rescaled.  Masked logits are -inf; a
// row with no valid key gets the uniform-weight result over all K keys
// (mean of V, max -1e9, lse -1e9 + ln K), as in the other kernels.
//
// Block masks (the tensorplay BlockMask page): the listed and full blocks of
// the workgroup's block row (kv_indices and full_kv_indices, read as a
// union, ids out of range ignored) are marked as bits in LDS; key tiles of
// unlisted blocks are skipped, and the causal mask_mod (query >= key)
// applies per element only on listed blocks that are not full (with 16-key
// blocks, a tile holds two, each listed, full or causal on its own).  Query
// blocks of 32 or 64 rows put 4 or 2 block rows in the 128 rows (each
// wave's 32 rows in one): the workgroup visits the union of their listed
// blocks, and a wave masks whole the tiles its own row does not list.  Their
// bitmaps share the LDS of the one-row ones: the union, then each row's
// listed and full bits, kMultiWords words apiece.
#include <math.h>

#include "triattn_internal.h"

namespace triattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kW = 4;         // waves per workgroup
constexpr int kQT = 32 * kW;  // query rows per workgroup
constexpr int kKT = 32;       // keys per tile
constexpr int kDT = 32;       // head dimension of the tiles (zero columns past D)
constexpr int kRow = kDT + 1;  // LDS row stride in floats (odd)
constexpr int kWords = static_cast<int>(kMaxKvBlocks / 32);  // one bitmap of kv blocks
// 32- or 64-row query blocks: up to kRows block rows per workgroup, whose
// union and per-row bitmaps share the LDS of two one-row bitmaps
constexpr int kRows = kQT / 32;
constexpr int kMultiWords = 2 * kWords / (1 + 2 * kRows);

__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// max / sum of the two lanes of a row (lane and lane ^ 32)
__device__ __forceinline__ float max2(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float sum2(float x) { return x + __shfl_xor(x, 32); }

__global__ __launch_bounds__(64 * kW) void fp32_fwd_kernel(Params p) {
    __shared__ float k_lds[kKT * kRow];
    __shared__ float v_lds[kKT * kRow];
    __shared__ uint32_t valid_word;  // bit i: key k0 + i of the tile valid
    __shared__ uint32_t block_bits[2 * kWords];
    uint32_t* const listed_bits = block_bits;
    uint32_t* const full_bits = block_bits + kWords;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int64_t n_qt = (p.Q + kQT - 1) / kQT;
    const int64_t g = blockIdx.x / n_qt;  // (b, n, h)
    const int64_t q0 = (blockIdx.x % n_qt) * kQT;
    const int64_t h = g % p.H, n = (g / p.H) % p.N, b = g / (p.H * p.N);
    const int64_t D = p.D;
    // Rows: the (b, n, h) slices (row strides D), or for packed sequences
    // sequence b's rows of the packed tensors (row strides q_rs / kv_rs, head
    // h at column h D); Q and K are then that sequence's row counts.
    const bool varlen = p.mask_kind == kMaskVarlen;
    int64_t Q = p.Q, K = p.K, q_rs = D, kv_rs = D;
    const float* qb = static_cast<const float*>(p.q) + g * p.Q * D;
    const float* kb = static_cast<const float*>(p.k) + g * p.K * D;
    const float* vb = static_cast<const float*>(p.v) + g * p.K * D;
    int64_t q_first = 0;
    if (varlen) {
        const SeqRows sr = seq_rows(p, b);
        Q = sr.nq;
        K = sr.nk;
        q_first = sr.q0;
        q_rs = p.q_rs;
        kv_rs = p.kv_rs;
        qb = static_cast<const float*>(p.q) + sr.q0 * q_rs + h * D;
        kb = static_cast<const float*>(p.k) + sr.k0 * kv_rs + h * D;
        vb = static_cast<const float*>(p.v) + sr.k0 * kv_rs + h * D;
        if (q0 >= Q) return;  // the whole workgroup is past this sequence
    }
    const int64_t row = q0 + 32 * wave + col;  // this lane's query
    const bool row_ok = row < Q;
    const float* brow = p.bias && !varlen && row_ok ? p.bias + ((b * p.H + h) * Q + row) * K : nullptr;
    const uint8_t* dense = p.mask_kind == TRIATTN_MASK_DENSE ? p.dense + (b * p.N + n) * K : nullptr;

    int64_t limit = K;  // keys >= limit are never valid
    if (p.mask_kind == TRIATTN_MASK_KV_LENGTHS && p.kv_lengths) {
        const int64_t len = p.kv_lengths[b * p.N + n];
        limit = len < 0 ? 0 : (len > K ? K : len);
    }
    // causal packed sequences: key j <= row (no row of the workgroup sees
    // a key past its last row)
    const bool seq_causal = varlen && p.causal;
    if (seq_causal) limit = limit < q0 + kQT ? limit : q0 + kQT;
    const int64_t n_tiles = (limit + kKT - 1) / kKT;

    // the block row(s) of the workgroup: listed and full blocks as bits
    const bool block_kind = p.mask_kind == TRIATTN_MASK_BLOCK;
    const bool multi = block_kind && p.q_block < kQT;  // 32- or 64-row query blocks
    const int wrow = multi ? static_cast<int>(32 * wave / p.q_block) : 0;
    uint32_t* const my_listed = multi ? block_bits + kMultiWords * (1 + wrow) : listed_bits;
    uint32_t* const my_full = multi ? block_bits + kMultiWords * (1 + kRows + wrow) : full_bits;
    if (block_kind) {  // uniform over the workgroup
        const int words = static_cast<int>((p.n_kv_blocks + 31) / 32);
        const int clear = multi ? (1 + 2 * kRows) * kMultiWords : 2 * kWords;
        for (int i = tid; i < clear; i += 64 * kW) {
            // (one-row bitmaps: only the words of n_kv_blocks)
            if (multi || i % kWords < words) block_bits[i] = 0u;
        }
        __syncthreads();
        const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
        auto mark = [&](uint32_t* bits, const int32_t* counts, const int32_t* ids, int64_t width,
                        int64_t list_row) {
            int64_t cnt = counts[list_row];
            cnt = cnt < 0 ? 0 : (cnt > width ? width : cnt);
            for (int64_t j = tid; j < cnt; j += 64 * kW) {
                const int64_t id = ids[list_row * width + j];
                if (id >= 0 && id < p.n_kv_blocks) atomicOr(&bits[id >> 5], 1u << (id & 31));
            }
        };
        const int rows = multi ? static_cast<int>(kQT / p.q_block) : 1;
        for (int r = 0; r < rows; ++r) {
            const int64_t qrow_blk = q0 / p.q_block + r;
            if (qrow_blk >= p.n_q_rows) break;  // rows past Q
            const int64_t list_row = inst * p.n_q_rows + qrow_blk;
            uint32_t* const rl = multi ? block_bits + kMultiWords * (1 + r) : listed_bits;
            uint32_t* const rf = multi ? block_bits + kMultiWords * (1 + kRows + r) : full_bits;
            // (with several rows, listed_bits is their union)
            mark(rl, p.kv_num_blocks, p.kv_indices, p.max_blocks, list_row);
            if (multi) mark(listed_bits, p.kv_num_blocks, p.kv_indices, p.max_blocks, list_row);
            if (p.full_kv_num_blocks) {
                mark(rf, p.full_kv_num_blocks, p.full_kv_indices, p.full_max_blocks, list_row);
                mark(rl, p.full_kv_num_blocks, p.full_kv_indices, p.full_max_blocks, list_row);
                if (multi)
                    mark(listed_bits, p.full_kv_num_blocks, p.full_kv_indices, p.full_max_blocks,
                         list_row);
            }
        }
        __syncthreads();
    }
    // 16-key blocks: tile t holds blocks 2t and 2t + 1
    const bool kv16 = block_kind && p.kv_block == 16;
    const int64_t tiles_per_block = block_kind && !kv16 ? p.kv_block / kKT : 1;
    auto bit = [](const uint32_t* bits, int64_t i) { return ((bits[i >> 5] >> (i & 31)) & 1u) != 0; };

    // Q^T operand: dims 16 half .. 16 half + 15 of the row (0 past D)
    float qv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t d = 16 * half + 4 * j;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (row_ok && d < D) x = *reinterpret_cast<const f32x4*>(qb + row * q_rs + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[4 * j + e] = x[e];
    }

    f32x16 o = {};
    float m = -INFINITY;  // running max of the valid logits of the row
    float l = 0.f;        // this lane's half of the running sum
    // staging: thread t copies 4 floats (chunk t % 8) of key row t / 8
    const int st_key = tid >> 3, st_c = tid & 7;
    for (int64_t t = 0; t < n_tiles; ++t) {
        const int64_t k0 = t * kKT;
        // keys of the tile listed for this wave's block row, and keys under
        // the causal mask_mod (listed, not full)
        uint32_t mine_w = ~0u, causal_w = 0u;
        if (block_kind) {
            const bool causal_mod = p.mask_mod == TRIATTN_MOD_CAUSAL;
            if (kv16) {
                const int64_t b0 = 2 * t;
                // (uniform: no barrier skipped unevenly)
                if (!bit(listed_bits, b0) && !bit(listed_bits, b0 + 1)) continue;
                const bool l0 = bit(my_listed, b0), l1 = bit(my_listed, b0 + 1);
                mine_w = (l0 ? 0x0000ffffu : 0u) | (l1 ? 0xffff0000u : 0u);
                if (causal_mod)
                    causal_w = (l0 && !bit(my_full, b0) ? 0x0000ffffu : 0u) |
                               (l1 && !bit(my_full, b0 + 1) ? 0xffff0000u : 0u);
            } else {
                const int64_t blk = t / tiles_per_block;
                if (!bit(listed_bits, blk)) continue;  // (uniform: no barrier skipped unevenly)
                mine_w = bit(my_listed, blk) ? ~0u : 0u;
                causal_w = causal_mod && !bit(my_full, blk) ? ~0u : 0u;
            }
        }
        if (seq_causal) causal_w = ~0u;
        __syncthreads();  // the previous tile is no longer read
        {
            const int64_t key = k0 + st_key;
            const int64_t d = 4 * st_c;
            f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (key < K && d < D) {
                kx = *reinterpret_cast<const f32x4*>(kb + key * kv_rs + d);
                vx = *reinterpret_cast<const f32x4*>(vb + key * kv_rs + d);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k_lds[st_key * kRow + 4 * st_c + e] = kx[e];
                v_lds[st_key * kRow + 4 * st_c + e] = vx[e];
            }
        }
        if (wave == 0) {
            const int64_t key = k0 + lane;
            const bool ok = lane < kKT && key < limit && (!dense || dense[key] != 0);
            const uint64_t bits = __ballot(ok);
            if (lane == 0) valid_word = static_cast<uint32_t>(bits);
        }
        __syncthreads();
        const uint32_t vw = valid_word;

        // S^T of the tile
        f32x16 s = {};
#pragma unroll
        for (int st = 0; st < 16; ++st) s = mma(k_lds[col * kRow + st + 16 * half], qv[st], s);

        // logits, tile max
        float z[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = 8 * (r / 4) + 4 * half + (r % 4);
            const bool ok = (((vw & mine_w) >> kr) & 1u) && (((causal_w >> kr) & 1u) == 0u || row >= k0 + kr);
            const float bias = brow && ok ? brow[k0 + kr] : 0.f;
            z[r] = ok ? fmaf(s[r], p.scale, bias) : -INFINITY;
            tmax = fmaxf(tmax, z[r]);
        }
        const float m_new = fmaxf(m, max2(tmax));
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = expf(m - m_use);
        float psum = 0.f;
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            pr[r] = expf(z[r] - m_use);  // 0 for a masked key
            psum += pr[r];
        }
        l = l * alpha + psum;
        o *= alpha;
        m = m_new;

        // O^T += V^T . P^T
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = 8 * (r / 4) + 4 * half + (r % 4);
            o = mma(v_lds[kr * kRow + col], pr[r], o);
        }
    }

    const float l_tot = sum2(l);
    const bool dead = m == -INFINITY;
    // a row with no valid key: the mean of V over all K keys (every lane
    // sums the columns it stores)
    float mean[16];
    if (dead) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mean[r] = 0.f;
        for (int64_t key = 0; key < K; ++key) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int64_t d = 8 * gq + 4 * half;
                if (d < D) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(vb + key * kv_rs + d);
#pragma unroll
                    for (int e = 0; e < 4; ++e) mean[4 * gq + e] += x[e];
                }
            }
        }
        const float inv = K > 0 ? 1.0f / static_cast<float>(K) : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) mean[r] *= inv;
    }
    if (!row_ok) return;
    const int64_t ridx = varlen ? (q_first + row) * p.H + h : g * p.Q + row;  // (row, head) index
    float* orow = static_cast<float*>(p.out) + ridx * D;
    const float inv_l = dead ? 0.f : 1.0f / l_tot;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
        const int64_t d = 8 * gq + 4 * half;
        if (d < D) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = dead ? mean[4 * gq + e] : o[4 * gq + e] * inv_l;
            *reinterpret_cast<f32x4*>(orow + d) = x;
        }
    }
    if (half == 0) {
        if (p.lse) p.lse[ridx] = dead ? kMaskedLogit + (K > 0 ? logf(static_cast<float>(K)) : 0.f)
                                      : m + logf(l_tot);
        if (p.mx) p.mx[ridx] = dead ? kMaskedLogit : m;
    }
}

}  // namespace

bool fp32_mfma_supports(const Params& p) {
    if (p.mask_kind != TRIATTN_MASK_NONE && p.mask_kind != TRIATTN_MASK_KV_LENGTHS &&
        p.mask_kind != TRIATTN_MASK_DENSE && p.mask_kind != TRIATTN_MASK_BLOCK &&
        p.mask_kind != kMaskVarlen)
        return false;
    // a workgroup's 128 rows in one block row, or 2 or 4 rows of 64 / 32
    // (their bitmaps hold kMultiWords x 32 kv blocks); whole 32-key tiles
    // per block
    if (p.mask_kind == TRIATTN_MASK_BLOCK) {
        if ((p.kv_block % kKT != 0 && p.kv_block != 16) || p.n_kv_blocks > kMaxKvBlocks) return false;
        if (p.q_block % kQT != 0 &&
            ((p.q_block != 32 && p.q_block != 64) || p.n_kv_blocks > kMultiWords * 32))
            return false;
    }
    if (p.D < 4 || p.D > kDT || p.D % 4 != 0 || p.bias16) return false;
    // 16-byte loads of Q, K and V rows and stores of O rows
    const uintptr_t al = reinterpret_cast<uintptr_t>(p.q) | reinterpret_cast<uintptr_t>(p.k) |
                         reinterpret_cast<uintptr_t>(p.v) | reinterpret_cast<uintptr_t>(p.out);
    return al % 16 == 0;
}

hipError_t launch_fp32_mfma(const Params& p, hipStream_t stream) {
    const int64_t groups = p.B * p.N * p.H * ((p.Q + kQT - 1) / kQT);
    if (groups > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fp32_fwd_kernel, dim3(static_cast<unsigned>(groups)), dim3(64 * kW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace triattn
