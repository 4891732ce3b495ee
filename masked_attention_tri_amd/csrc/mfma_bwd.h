// MFMA backward kernels for bf16 / fp16 inputs, D in {32, 64, 128}.
//
// The forward (cuequivariance_torch.triangle_attention page, the defining
// equation) per (b, n, h, q) row is O_q = sum_k P_qk V_k with P the softmax of
// z_qk = s Q_q.K_k + B_qk over the valid keys.  Its gradient, given dO:
//
//   dV_k  = sum_q P_qk dO_q
//   dz_qk = P_qk (dO_q.V_k - Delta_q),   Delta_q = dO_q.O_q
//   dQ_q  = s sum_k dz_qk K_k,   dK_k = s sum_q dz_qk Q_q,   dB_qk = sum_n dz_qk
//
// with P rebuilt from the forward's lse (P = exp(z - lse)).  A row whose
// forward max is the -1e9 replacement had no valid key: its P is 1/K for
// every key and it passes nothing to Q, K or the bias.
//
// Each gradient is a sum over a different axis (dQ over keys, dK and dV over
// queries, dB over n), so each gets a kernel that keeps its own sum in
// registers and recomputes z, dP, P and dz for its tile; nothing is summed
// with atomics and every sum runs in a fixed order.  Four launches:
//
//   bwd_rows_kernel   Delta and -lse log2 e of every row, and per 32-row tile
//                     the number of rows with no valid key, into the
//                     workspace (260 bytes per 32-row tile).
//   bwd_dkdv_kernel   one workgroup per (b, n, h, 128 keys); K and V rows in
//                     registers; 32-row query tiles of Q, dO and the row data
//                     by LDS DMA.
//   bwd_dbias_kernel  one workgroup per (b, h, 128 queries and 128 keys (64 x
//                     64 at D = 128), range of n), walking n: the bias block stays in
//                     registers, Q, dO, K and V of each n arrive by LDS DMA,
//                     dB accumulates in registers; the ranges' sums are added
//                     in order by bwd_dbias_combine_kernel.
//   bwd_dq_kernel     one workgroup per (b, n, h, 128 queries), the forward's
//                     layout: Q and dO rows in registers, 32-key tiles of K, V
//                     and the bias by LDS DMA.
//
// Contractions run on v_mfma_f32_32x32x16_{bf16,f16}; P and dz enter the
// accumulating ones rounded to the input type.  Tiles that are read both in
// row order (an MFMA operand of z or dP) and transposed (ds_read_b64_tr_b16,
// the operand of the accumulating product) share one XOR swizzle that keeps
// both reads free of bank conflicts (BGeo::f).
#pragma once

#include <math.h>

#include "mfma_common.h"

namespace triattn {
namespace {

using namespace tile;

// LDS geometry of a 32-row tile of D elements per row.
template <int D>
struct BGeo {
    static constexpr int rowBytes = 2 * D;
    static constexpr int chunks = D / 8;  // 16-byte chunks per row
    static constexpr int tileBytes = 32 * rowBytes;
    static constexpr int tileDma = tileBytes / 1024;  // DMA instructions per tile
    static_assert(tileDma * 1024 == tileBytes, "whole DMA instructions per tile");
    // Chunk c of row r is stored at c ^ f(r).  Row reads (16 bytes per lane,
    // 16 consecutive rows at one chunk per LDS cycle): the rows sharing one
    // bank group must get distinct f.  Transposed reads (8 bytes per lane; 32
    // lanes read 4 consecutive rows r0..r0+3, r0 a multiple of 4, at 4
    // adjacent chunks 4a..4a+3): rows sharing one bank group must land in
    // distinct 4-chunk groups.  D = 32 (4 rows per 256 bytes): rows r, r+4,
    // r+8, r+12 share banks and f = r / 4 maps them to 0..3; transposed reads
    // take one whole row per bank quarter.  D = 64 (2 rows per 256 bytes): f is a
    // bijection on the even (and on the odd) rows of 16, and rows 4m and
    // 4m+2 differ in bit 2.  D = 128: f is a bijection on 16 rows whose bits
    // 2-3 differ within each aligned group of 4 rows.  f depends on r % 16
    // only.
    static __device__ __forceinline__ int f(int r) {
        static_assert(D == 32 || D == 64 || D == 128, "swizzles defined");
        if (D == 32) return (r >> 2) & 3;
        if (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
        return ((r & 3) << 2) | ((r >> 2) & 3);
    }
    // Byte offset (within a tile) that lane l (row l % 32, chunk half) reads
    // for MFMA k-step st: 16 bytes, elements 16 st + 8 half .. + 7 of row
    // l % 32.  XOR with 32 st selects the step.
    static __device__ __forceinline__ int row_base(int col, int half) {
        return col * rowBytes + 16 * (half ^ f(col));
    }
    // Transposed read (ds_read_b64_tr_b16): lane s names row 8u + 4 half +
    // (s % 16) / 4 and byte 8 (s % 2) of chunk 2 ((s / 16) % 2) + (s % 4) / 2
    // (+ 4 per 32-column block, an XOR with 64 jb); it then receives column
    // 32 jb + s % 32 of the 4 rows of its slots.  Rows 16 st further use the
    // same swizzle, so step st adds 16 st rows.
    static __device__ __forceinline__ int tr_base(int lane, int u) {
        const int r = 8 * u + 4 * (lane >> 5) + ((lane & 15) >> 2);
        const int chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        return r * rowBytes + 16 * (chunk ^ f(r)) + 8 * (lane & 1);
    }
    // Source offset (within a tile in memory, rows of D elements) of DMA slot
    // s = 64 i + lane of instruction i of a tile.
    static __device__ __forceinline__ uint32_t dma_src(int i, int lane) {
        const int s = 64 * i + lane;
        const int r = s / chunks, c = s % chunks;
        return static_cast<uint32_t>(r * rowBytes + 16 * (c ^ f(r)));
    }
    // The same for rows of dn <= D elements in memory (dn a multiple of 8):
    // a source chunk at or past dn / 8 reads at kNoTile and lands as zeros
    // (with a tile offset added the sum stays in [2^31, 2^32), past every
    // slice).  With dn = D it is dma_src.
    static __device__ __forceinline__ uint32_t dma_src(int i, int lane, int dn) {
        const int s = 64 * i + lane;
        const int r = s / chunks, c = s % chunks;
        const int sc = c ^ f(r);
        return 8 * sc < dn ? static_cast<uint32_t>(r * 2 * dn + 16 * sc) : kNoTile;
    }
};

// Eight elements of a row at column c0 (a multiple of 8) of a row of dn
// elements, zeros at and past dn; the load is unconditional (from the row's
// first columns there) so that several stay in flight together.
template <typename V, typename T>
__device__ __forceinline__ V load8_or_zero(const T* row, int c0, int dn) {
    const bool in_row = c0 < dn;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(row + (in_row ? c0 : 0));
    return __builtin_bit_cast(V, in_row ? raw : u32x4{0u, 0u, 0u, 0u});
}

// The A operand of an accumulating product from a tile: rows 16 st + 4 half
// + 0..3 and 16 st + 8 + 4 half + 0..3 of column 32 jb + lane % 32, i.e. the
// order in which a lane holds P (or dz) of its 16 rows in registers 8 st ..
// 8 st + 7.
template <typename V8, int D>
__device__ __forceinline__ V8 tr_operand(const lds_char* tile, int tr0, int tr1, int jb, int st) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(tile + (tr0 ^ (64 * jb)) + 16 * st * BGeo<D>::rowBytes));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(tile + (tr1 ^ (64 * jb)) + 16 * st * BGeo<D>::rowBytes));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(V8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

template <typename V8>
__device__ __forceinline__ V8 row_operand(const lds_char* tile, int base, int st) {
    return __builtin_bit_cast(V8, *reinterpret_cast<const lds_u32x4*>(tile + (base ^ (32 * st))));
}

// Round four fp32 values to T and store them as 8 bytes.
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
    T v[4] = {static_cast<T>(a), static_cast<T>(b), static_cast<T>(c), static_cast<T>(d)};
    *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, v);
}

// ---- per-row data -----------------------------------------------------------
// Per (b, n, h) slice and 32-row tile t, 64 floats at rows + (slice nT + t) 64:
// -Delta of the tile's 32 rows (Delta_q = dO_q . O_q, fp32 products of the
// stored values), then -lse_q log2 e (NaN when the forward's max of row q is
// the -1e9 replacement: no valid key); rows past Q hold 0 and -inf.  Then,
// after all tiles, tile_dead[slice nT + t] = rows of tile t with no valid key.
// Workspace bytes: 260 per (slice, tile) (bwd_rows_bytes).  One workgroup of
// 32 (D / 8) threads per tile: thread (r, c) takes the 16-byte chunk c of row
// r; shuffles sum the D / 8 partial products.
template <typename T, int D, bool PAD>
__global__ __launch_bounds__(4 * D) void bwd_rows_kernel(Params p, BwdParams g, float* rows,
                                                         uint32_t* tile_dead) {
    using v8 = typename Mma<T>::v8;
    constexpr int kC = D / 8;
    const int64_t n_t = (p.Q + 31) / 32;
    const int64_t total = p.B * p.N * p.H * n_t;
    const int tid = threadIdx.x, r = tid / kC, c = tid % kC;
    for (int64_t w = blockIdx.x; w < total; w += gridDim.x) {
        const int64_t bnh = w / n_t, q = 32 * (w % n_t) + r;
        const bool in = q < p.Q;
        float acc = 0.f, lse = 0.f, mx = 0.f;
        if (in) {
            // the row's lse and max are loaded with its O and dO (every
            // thread of the row: one request per row), not after the sum
            const int64_t i = bnh * p.Q + q;
            lse = g.lse[i];
            mx = g.mx[i];
            // (rows of Dn elements; with PAD the columns past Dn are zeros)
            const int Dn = PAD ? static_cast<int>(p.D) : D;
            const int64_t off = i * Dn;
            const v8 go = load8_or_zero<v8>(static_cast<const T*>(g.dout) + off, 8 * c, Dn);
            const v8 o = load8_or_zero<v8>(static_cast<const T*>(g.out) + off, 8 * c, Dn);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(static_cast<float>(go[e]), static_cast<float>(o[e]), acc);
        }
#pragma unroll
        for (int s = 1; s < kC; s <<= 1) acc += __shfl_xor(acc, s);
        const bool dead = in && mx == kMaskedLogit;
        if (c == 0) {
            rows[w * 64 + r] = -acc;
            rows[w * 64 + 32 + r] = !in ? -INFINITY : dead ? __builtin_nanf("") : -lse * kLog2e;
        }
        const int cnt = __syncthreads_count(dead && c == 0);  // one vote per row
        if (tid == 0) tile_dead[w] = static_cast<uint32_t>(cnt);
    }
}

// Lane i of the result: bit j set when 32-row tile 32 i + j of the slice has
// a row with no valid key (nT <= 2048 tiles).
__device__ __forceinline__ uint32_t load_dead_word(const uint32_t* td, int nT, int lane) {
    uint32_t word = 0;
    for (int t0 = 0; t0 < nT; t0 += 64) {
        const int t = t0 + lane;
        const uint64_t bits = __ballot(t < nT && td[t] != 0u);
        const int i = t0 >> 5;
        word = lane == i ? static_cast<uint32_t>(bits) : word;
        word = lane == i + 1 ? static_cast<uint32_t>(bits >> 32) : word;
    }
    return word;
}

// Workgroup id -> logical id such that each of the 8 XCDs walks a contiguous
// range of the logical order (consecutive workgroup ids go round the XCDs).
__device__ __forceinline__ int64_t xcd_order(int64_t w, int64_t n_wg) {
    const int64_t xcd = w % kXcds, slot = w / kXcds;
    const int64_t per = n_wg / kXcds, rem = n_wg % kXcds;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Waves per SIMD the register budget must allow: two for D <= 64, one for
// D = 128 (whose operands and sums need more than 256 VGPRs).
template <int D>
constexpr int bwd_waves_per_simd() {
    return D <= 64 ? 2 : 1;
}

// Largest number of query blocks of a block-sparse mask the dK/dV kernel
// takes (one bit per block and kv block of the workgroup in LDS).
constexpr int64_t kMaxQBlocks = 2048;

// Bias paths of the backward kernels.
enum BwdBias { kBNone = 0, kBLds = 1, kBScalar = 2 };

// ---- dK, dV -----------------------------------------------------------------
// One workgroup of 4 waves per (b, n, h, 128 keys); wave w owns keys 32 w ..
// 32 w + 31, lane l key 32 w + l % 32, whose K and V rows it holds as MFMA B
// operands.  Per 32-row query tile (shared by the workgroup, LDS DMA two
// tiles ahead in rings of three):
//   z  = Q K^T + C          A = Q rows, C = the bias block (rows = queries)
//   dP = dO V^T - Delta     A = dO rows, -Delta the initial accumulator
// leave lane l with its key and 16 queries (register r: query 8 (r / 4) +
// 4 (l / 32) + r % 4); P and dz are formed there and
//   dV^T += dO^T P,  dK^T += Q^T dz     A = dO^T, Q^T by transposed reads
// take them as B operands.  The bias block of each wave (32 queries x 32
// keys, fp32) arrives by DMA into the wave's own LDS region, refilled with
// the next tile's block as soon as it has been read; its rows are stored
// permuted (row r at r ^ ((r >> 2) & 1)) so that the two wave halves, which
// read rows 4 apart, hit opposite bank halves.  Per-row Delta and lse come
// from the row data by a 64-byte DMA per wave.
//
// Masks: kv_lengths and dense masks make whole lanes (keys) invalid; block
// lists make whole (query tile, wave) pairs invalid, read from per-kv-block
// bitmaps of the query blocks that list them (built in LDS from the kv lists
// at the start, the lists transposed); causal partial blocks mask per
// element.  A tile where every element is valid and no row lacks a valid key
// takes the plain path; otherwise each element selects.  Tiles that no wave
// needs (unlisted and without rows lacking a valid key) are skipped.
template <typename T, int D, int KIND, int BIAS, bool EXACT, bool PAD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>()))) void bwd_dkdv_kernel(
    Params p, BwdParams g, const float* rows, const uint32_t* tile_dead) {
    using M = Mma<T>;
    using v8 = typename M::v8;
    using Ge = BGeo<D>;
    constexpr bool kBlock = KIND == TRIATTN_MASK_BLOCK;
    constexpr bool kDense = KIND == TRIATTN_MASK_DENSE;
    constexpr int kRingDma = 2 * Ge::tileDma / 4;  // Q and dO DMAs per wave and tile
    constexpr int kInFlight = kRingDma + 1;        // and one row-data DMA
    constexpr int kQWords = kBlock ? static_cast<int>(kMaxQBlocks / 32) : 1;
    __shared__ __attribute__((aligned(1024))) char q_lds0[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char q_lds1[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char q_lds2[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char g_lds0[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char g_lds1[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char g_lds2[Ge::tileBytes];
    __shared__ __attribute__((aligned(256))) char r_lds0[256];
    __shared__ __attribute__((aligned(256))) char r_lds1[256];
    __shared__ __attribute__((aligned(256))) char r_lds2[256];
    __shared__ __attribute__((aligned(1024))) char b_lds[BIAS == kBLds ? 4 * kBiasWaveBytes : 16];
    // block lists: per kv block of the workgroup, the query blocks listing it
    __shared__ uint32_t q_listed[kBlock ? 4 : 1][kQWords];
    __shared__ uint32_t q_full[kBlock ? 4 : 1][kQWords];
    __shared__ uint32_t q_any[kQWords];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    // ---- workgroup -> (b, h, n, key block), XCD-contiguous -----------------
    const int64_t n_kb = (p.K + 127) / 128;
    const int64_t lid = xcd_order(blockIdx.x, gridDim.x);
    const int64_t kb = lid % n_kb;
    const int64_t n = (lid / n_kb) % p.N;
    const int64_t h = (lid / (n_kb * p.N)) % p.H;
    const int64_t b = lid / (n_kb * p.N * p.H);
    const int64_t bnh = (b * p.N + n) * p.H + h;
    const int K = static_cast<int>(p.K), Q = static_cast<int>(p.Q);
    const int nT = (Q + 31) / 32;
    const int kw0 = static_cast<int>(kb) * 128;
    const int kw = kw0 + 32 * wave;  // this wave's first key
    const int key = kw + col;        // this lane's key

    // ---- key validity -------------------------------------------------------
    int lim = K;
    if (KIND == TRIATTN_MASK_KV_LENGTHS && p.kv_lengths) {
        const int64_t len = p.kv_lengths[b * p.N + n];
        lim = len < 0 ? 0 : (len > K ? K : static_cast<int>(len));
    }
    bool lane_ok = key < lim;
    if constexpr (kDense) lane_ok = lane_ok && p.dense[(b * p.N + n) * p.K + key] != 0;
    // every stored key of the wave valid / some key valid
    const bool wave_clean = __ballot(key < K && !lane_ok) == 0;
    const bool wave_any = __ballot(lane_ok) != 0;
    const float inv_k = 1.0f / static_cast<float>(K);

    const uint32_t dead_word = load_dead_word(tile_dead + bnh * nT, nT, lane);
    const bool slice_dead = __ballot(dead_word != 0u) != 0;
    auto tile_has_dead = [&](int t) -> bool {
        return (static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dead_word), t >> 5)) >>
                (t & 31)) & 1u;
    };

    // Dn: the head dimension of the data, D that of the tiles (with PAD, Dn <
    // D and a multiple of 8: columns past Dn enter as zeros and are not stored)
    const int Dn = PAD ? static_cast<int>(p.D) : D;
    T* dkb = static_cast<T*>(g.dk) + bnh * p.K * Dn;
    T* dvb = static_cast<T*>(g.dv) + bnh * p.K * Dn;
    // Keys past the length with every row having a valid key: nothing to add.
    if (!kBlock && kw0 >= lim && !slice_dead) {
        if (key < K) {
#pragma unroll
            for (int d = 0; d < D; d += 4) {
                if (d < Dn) {  // (not a padding column)
                    *reinterpret_cast<u32x2*>(dkb + static_cast<int64_t>(key) * Dn + d) = u32x2{0u, 0u};
                    *reinterpret_cast<u32x2*>(dvb + static_cast<int64_t>(key) * Dn + d) = u32x2{0u, 0u};
                }
            }
        }
        return;
    }

    // ---- block lists, transposed: query blocks listing each kv block --------
    int64_t kvb_lo = 0;
    int slot = 0;
    if constexpr (kBlock) {
        kvb_lo = kw0 / p.kv_block;
        const int64_t kvb_hi = min(static_cast<int64_t>(kw0 + 127) / p.kv_block, p.n_kv_blocks - 1);
        const int words = static_cast<int>((p.n_q_rows + 31) / 32);
        for (int i = tid; i < 4 * words; i += 256) {
            q_listed[i / words][i % words] = 0u;
            q_full[i / words][i % words] = 0u;
        }
        __syncthreads();
        const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
        auto scan = [&](const int32_t* counts, const int32_t* ids, int64_t width, bool full) {
            const int64_t total = p.n_q_rows * width;
            for (int64_t e = tid; e < total; e += 256) {
                const int64_t i = e / width, j = e - (e / width) * width;
                const int64_t row = inst * p.n_q_rows + i;
                int64_t cnt = counts[row];
                cnt = cnt < 0 ? 0 : (cnt > width ? width : cnt);
                if (j >= cnt) continue;
                const int64_t id = ids[row * width + j];
                if (id < kvb_lo || id > kvb_hi) continue;
                const int s = static_cast<int>(id - kvb_lo);
                atomicOr(&q_listed[s][i >> 5], 1u << (i & 31));
                if (full) atomicOr(&q_full[s][i >> 5], 1u << (i & 31));
            }
        };
        scan(p.kv_num_blocks, p.kv_indices, p.max_blocks, false);
        if (p.full_kv_num_blocks) scan(p.full_kv_num_blocks, p.full_kv_indices, p.full_max_blocks, true);
        __syncthreads();
        for (int i = tid; i < words; i += 256) q_any[i] = q_listed[0][i] | q_listed[1][i] | q_listed[2][i] | q_listed[3][i];
        __syncthreads();
        slot = static_cast<int>(min(static_cast<int64_t>(kw), p.K - 1) / p.kv_block - kvb_lo);
    }

    // ---- tile sequence -------------------------------------------------------
    // every tile, or (block lists) the tiles some wave needs: listed for one
    // of the workgroup's kv blocks, or holding a row with no valid key
    auto next_tile = [&](int t) -> int {
        const int c = t + 1;
        if (c >= nT) return -1;
        if constexpr (!kBlock) {
            return c;
        } else {
            int best = nT;
            const int64_t qb = static_cast<int64_t>(32 * c) / p.q_block;
            if (bit_set(q_any, qb)) {
                best = c;
            } else {
                const int64_t nb = next_set(q_any, qb + 1, p.n_q_rows);
                if (nb >= 0) best = static_cast<int>(nb * p.q_block / 32);
            }
            if (slice_dead) {
                for (int wd = c >> 5; wd * 32 < best && wd * 32 < nT; ++wd) {
                    uint32_t bits = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dead_word), wd));
                    if (wd == (c >> 5)) bits &= ~0u << (c & 31);
                    if (bits) {
                        best = min(best, 32 * wd + static_cast<int>(__builtin_ctz(bits)));
                        break;
                    }
                }
            }
            return best < nT ? best : -1;
        }
    };

    // ---- K, V rows of this lane's key (B operands) --------------------------
    v8 kop[D / 16], vop[D / 16];
    {
        const T* kr = static_cast<const T*>(p.k) + (bnh * p.K + (key < K ? key : K - 1)) * Dn;
        const T* vr = static_cast<const T*>(p.v) + (bnh * p.K + (key < K ? key : K - 1)) * Dn;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            v8 x = load8_or_zero<v8>(kr, 16 * st + 8 * half, Dn);
            if (EXACT) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = static_cast<T>(static_cast<float>(x[j]) * p.scale);
            }
            kop[st] = x;
            vop[st] = load8_or_zero<v8>(vr, 16 * st + 8 * half, Dn);
        }
    }
    const float c_exp = (EXACT ? 1.0f : p.scale) * kLog2e;  // exponent slope of Q.K + C
    const float inv_s = EXACT ? 1.0f : 1.0f / p.scale;      // bias -> units of Q.K

    // ---- DMA --------------------------------------------------------------
    const uint32_t slice_bytes = static_cast<uint32_t>(p.Q * Dn * sizeof(T));
    const u32x4 q_desc = make_desc(static_cast<const T*>(p.q) + bnh * p.Q * Dn, slice_bytes);
    const u32x4 g_desc = make_desc(static_cast<const T*>(g.dout) + bnh * p.Q * Dn, slice_bytes);
    const uint32_t mem_tile = static_cast<uint32_t>(32 * 2 * Dn);  // one tile of rows in memory
    const u32x4 r_desc = make_desc(rows + bnh * nT * 64, static_cast<uint32_t>(nT * 256));
    auto qbuf = [&](int x) { return (lds_char*)(x == 0 ? q_lds0 : x == 1 ? q_lds1 : q_lds2); };
    auto gbuf = [&](int x) { return (lds_char*)(x == 0 ? g_lds0 : x == 1 ? g_lds1 : g_lds2); };
    auto rbuf = [&](int x) { return (lds_char*)(x == 0 ? r_lds0 : x == 1 ? r_lds1 : r_lds2); };
    // instruction I = wave + 4 j of a tile: Q for I < tileDma, else dO
    uint32_t ring_src[kRingDma];
#pragma unroll
    for (int j = 0; j < kRingDma; ++j) ring_src[j] = Ge::dma_src((wave + 4 * j) % Ge::tileDma, lane, Dn);
    auto dma_ring = [&](int t, int x) {
        const uint32_t toff = t >= 0 ? static_cast<uint32_t>(t) * mem_tile : kNoTile;
#pragma unroll
        for (int j = 0; j < kRingDma; ++j) {
            const int I = wave + 4 * j;
            if (I < Ge::tileDma)
                dma16(q_desc, qbuf(x) + 1024 * I, ring_src[j] + toff);
            else
                dma16(g_desc, gbuf(x) + 1024 * (I - Ge::tileDma), ring_src[j] + toff);
        }
        // bytes 64 w .. 64 w + 63 of the tile's 256 bytes of row data
        const uint32_t roff = t >= 0 ? static_cast<uint32_t>(256 * t + 64 * wave + 16 * lane) : kNoTile;
        if (lane < 4) dma16(r_desc, rbuf(x) + 64 * wave, roff);
    };
    // bias block: instruction j, lane l fills stored row 8 j + l / 8 (source
    // row: the same permutation, an involution) at chunk l % 8
    const char* bplane = BIAS != kBNone ? reinterpret_cast<const char*>(p.bias + (b * p.H + h) * p.Q * p.K) : nullptr;
    const uint32_t bias_bytes = BIAS != kBNone ? static_cast<uint32_t>(p.Q * p.K * 4) : 0u;
    const u32x4 b_desc = make_desc(bplane, bias_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(bplane, bias_bytes);
    lds_char* const bias_lds = (lds_char*)b_lds + (BIAS == kBLds ? wave * kBiasWaveBytes : 0);
    uint32_t b_src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int sr = 8 * j + (lane >> 3);
        const int srow = sr ^ ((sr >> 2) & 1);
        b_src[j] = static_cast<uint32_t>((srow * K + kw) * 4 + 16 * (lane & 7));
    }
    auto dma_bias = [&](int t) {
        if constexpr (BIAS == kBLds) {
            const uint32_t toff = static_cast<uint32_t>(32 * t) * static_cast<uint32_t>(K) * 4u;
#pragma unroll
            for (int j = 0; j < 4; ++j) dma16(b_desc, bias_lds + 1024 * j, b_src[j] + toff);
        }
    };
    // register 4 c + i is query row 8 c + 4 half + i, stored at row
    // (8 c) + (4 half + i) ^ half (bit 2 of the row is half)
    int b_rd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b_rd[i] = ((4 * half + i) ^ half) * kBiasRowBytes + 4 * col;

    // per-lane offsets of the operand reads
    const int rrd = Ge::row_base(col, half);
    const int tr0 = Ge::tr_base(lane, 0), tr1 = Ge::tr_base(lane, 1);

    f32x16 ak[D / 32], av[D / 32];
#pragma unroll
    for (int jb = 0; jb < D / 32; ++jb) {
        ak[jb] = f32x16{};
        av[jb] = f32x16{};
    }

    auto compute = [&](int t, int x, auto dma) {
        const int q0 = 32 * t;
        const bool dead_t = tile_has_dead(t);
        bool listed = true, causal = false;
        if constexpr (kBlock) {
            const int64_t qb = static_cast<int64_t>(q0) / p.q_block;
            listed = bit_set(q_listed[slot], qb);
            const bool full = bit_set(q_full[slot], qb);
            if (listed && !full && p.mask_mod == TRIATTN_MOD_CAUSAL) {
                if (q0 + 31 < kw)
                    listed = false;  // every query of the tile is before every key
                else if (q0 < kw + 31)
                    causal = true;  // the diagonal crosses the tile
            }
        }
        if (!((listed && wave_any) || dead_t)) {
            dma();
            return;
        }
        const bool plain = listed && !causal && !dead_t && wave_clean && q0 + 32 <= Q;
        const lds_char* qt = qbuf(x);
        const lds_char* gt = gbuf(x);
        // -Delta (the initial accumulator of dP) and -lse log2 e of the 16
        // rows: 4 consecutive rows per c, one 16-byte read each
        const lds_char* rt = rbuf(x);
        f32x16 z, dp;
        float nl[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(rt + (8 * c + 4 * half) * 4);
            const f32x4 l = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(rt + 128 + (8 * c + 4 * half) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dp[4 * c + i] = a[i];
                nl[4 * c + i] = l[i];
            }
        }
        if constexpr (BIAS == kBLds) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    z[4 * c + i] = *reinterpret_cast<const __attribute__((address_space(3))) float*>(
                        bias_lds + b_rd[i] + 1024 * c);
        } else if constexpr (BIAS == kBScalar) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = q0 + 8 * (r / 4) + 4 * half + (r % 4);
                z[r] = bload32(b_rsrc, static_cast<uint32_t>((qr * K + key) * 4));
            }
        } else {
            z = f32x16{};
        }
        if (BIAS != kBNone && !EXACT) z *= inv_s;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) z = M::run(row_operand<v8>(qt, rrd, st), kop[st], z);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) dp = M::run(row_operand<v8>(gt, rrd, st), vop[st], dp);
        dma();
        v8 pop[2], zop[2];
        if (plain) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(z[r], c_exp, nl[r]));
                pop[r / 8][r % 8] = static_cast<T>(pr);
                zop[r / 8][r % 8] = static_cast<T>(pr * dp[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = q0 + 8 * (r / 4) + 4 * half + (r % 4);
                bool ok = lane_ok && listed && qr < Q;
                if (causal) ok = ok && qr >= key;
                const bool dead = nl[r] != nl[r];
                float pr = ok ? __builtin_amdgcn_exp2f(fmaf(z[r], c_exp, nl[r])) : 0.f;
                const float dz = ok && !dead ? pr * dp[r] : 0.f;
                pr = dead ? inv_k : pr;
                pop[r / 8][r % 8] = static_cast<T>(pr);
                zop[r / 8][r % 8] = static_cast<T>(dz);
            }
        }
#pragma unroll
        for (int jb = 0; jb < D / 32; ++jb)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                av[jb] = M::run(tr_operand<v8, D>(gt, tr0, tr1, jb, st), pop[st], av[jb]);
                ak[jb] = M::run(tr_operand<v8, D>(qt, tr0, tr1, jb, st), zop[st], ak[jb]);
            }
    };

    // ---- query-tile loop: ring position j holds tile t_j in buffers j % 3 ---
    int cur = [&] {
        if constexpr (!kBlock) return nT > 0 ? 0 : -1;
        else return next_tile(-1);
    }();
    int nxt = next_tile(cur);
    if (cur >= 0) {
        dma_bias(cur);
        dma_ring(cur, 0);
        dma_ring(nxt, 1);
        wait_vmem();
        __syncthreads();
    }
    auto step = [&](auto X) {
        constexpr int x = decltype(X)::value;
        const int nxt2 = nxt >= 0 ? __builtin_amdgcn_readfirstlane(next_tile(nxt)) : -1;
        // all but the previous position's ring DMAs have landed (in every
        // wave once all have passed the barrier, which also frees the buffers
        // refilled below)
        __builtin_amdgcn_s_waitcnt(kVmcntWait<kInFlight>());
        __syncthreads();
        compute(cur, x, [&] {
            if (nxt >= 0) {
                wait_lds();  // this wave's bias reads are done
                dma_bias(nxt);
            }
            dma_ring(nxt2, (x + 2) % 3);
        });
        cur = nxt;
        nxt = nxt2;
    };
    while (cur >= 0) {
        step(Par<0>{});
        if (cur < 0) break;
        step(Par<1>{});
        if (cur < 0) break;
        step(Par<2>{});
    }
    wait_vmem();  // no DMA outlives the workgroup

    // ---- epilogue: lane = key, register r = column 32 jb + 8 (r / 4) + 4 half + r % 4
    if (key >= K) return;
    T* dkr = dkb + static_cast<int64_t>(key) * Dn;
    T* dvr = dvb + static_cast<int64_t>(key) * Dn;
#pragma unroll
    for (int jb = 0; jb < D / 32; ++jb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int d0 = 32 * jb + 8 * c + 4 * half;
            if (d0 >= Dn) continue;  // a padding column
            store4(dkr + d0, ak[jb][4 * c] * p.scale, ak[jb][4 * c + 1] * p.scale,
                   ak[jb][4 * c + 2] * p.scale, ak[jb][4 * c + 3] * p.scale);
            store4(dvr + d0, av[jb][4 * c], av[jb][4 * c + 1], av[jb][4 * c + 2], av[jb][4 * c + 3]);
        }
}

// ---- dQ -----------------------------------------------------------------
// The forward kernel's layout: one workgroup of 4 waves per (b, n, h, 128
// query rows), wave w owning rows 32 w .. 32 w + 31 and lane l row 32 w + l %
// 32, whose Q (scaled by s when that is exact) and dO rows it holds as MFMA
// B operands; Delta = dO.O of the row is reduced from dO and O in the
// prologue, and -lse log2 e is a per-lane constant (-inf for a row with no
// valid key, so that its P and dz vanish).  Per 32-key tile (K and V by LDS
// DMA two tiles ahead in rings of three, the wave's 32 x 32 fp32 bias block
// by DMA into its own LDS region):
//   z^T  = K Q^T + C          A = K rows, C = the bias block (rows = queries)
//   dP^T = V dO^T - Delta     A = V rows, -Delta the initial accumulator
// leave lane l with its row and 16 keys; P and dz are formed there and
//   dQ^T += K^T dz^T    A = K^T by transposed reads of the same K tile
// takes dz as the B operand.  Masks as in the forward kernel: tiles past
// the length or not listed are not visited, element masks only where a tile
// needs one.
// dQ kernel variant (a template value, not a mask kind of the calls) of
// block masks with 32- or 64-row query blocks: 4 or 2 block rows per
// 128-row workgroup, each wave's 32 rows in one.  Their bitmaps share the
// LDS of the one-row ones: the union of the rows' listed kv blocks (the
// tiles visited), then each row's listed and full blocks, kMultiWords
// words apiece.
constexpr int kBwdBlockRows = 5;

template <typename T, int D, int KIND, int BIAS, bool EXACT, bool PAD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>()))) void bwd_dq_kernel(
    Params p, BwdParams g) {
    using M = Mma<T>;
    using v8 = typename M::v8;
    using Ge = BGeo<D>;
    constexpr bool kBlock = KIND == TRIATTN_MASK_BLOCK || KIND == kBwdBlockRows;
    constexpr bool kMultiRow = KIND == kBwdBlockRows;
    constexpr bool kDense = KIND == TRIATTN_MASK_DENSE;
    constexpr int kKvDma = 2 * Ge::tileDma / 4;  // K and V DMAs per wave and tile
    constexpr int kWords = static_cast<int>(kMaxKvBlocks / 32);
    __shared__ __attribute__((aligned(1024))) char k_lds0[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds2[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds2[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char b_lds[BIAS == kBLds ? 4 * kBiasWaveBytes : 16];
    __shared__ uint32_t block_bits[kBlock ? 2 * kWords : 1];
    uint32_t* const listed_bits = block_bits;
    uint32_t* const full_bits = block_bits + kWords;
    auto row_listed = [&](int r) { return block_bits + kMultiWords * (1 + r); };
    auto row_full = [&](int r) { return block_bits + kMultiWords * (1 + kRowsMulti + r); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    // ---- workgroup -> (b, h, n, q tile), XCD-contiguous; q tiles of one
    // (b, n, h) alternate between the ends (balances causal block masks)
    const int64_t n_qt = (p.Q + 127) / 128;
    const int64_t lid = xcd_order(blockIdx.x, gridDim.x);
    const int64_t qr = lid % n_qt;
    const int64_t qt0 = (qr & 1) ? n_qt - 1 - qr / 2 : qr / 2;
    const int64_t qt = ((lid / n_qt) & 1) ? n_qt - 1 - qt0 : qt0;
    const int64_t n = (lid / n_qt) % p.N;
    const int64_t h = (lid / (n_qt * p.N)) % p.H;
    const int64_t b = lid / (n_qt * p.N * p.H);
    const int64_t bnh = (b * p.N + n) * p.H + h;
    const int K = static_cast<int>(p.K), Q = static_cast<int>(p.Q);
    const int q0 = static_cast<int>(qt) * 128;
    const int q0w = q0 + 32 * wave;
    const int qrow = q0w + col;
    const bool row_ok = qrow < Q;
    const int qload = row_ok ? qrow : Q - 1;

    // ---- visited key tiles -------------------------------------------------
    int limit = K;
    if (KIND == TRIATTN_MASK_KV_LENGTHS && p.kv_lengths) {
        const int64_t len = p.kv_lengths[b * p.N + n];
        limit = len < 0 ? 0 : (len > K ? K : static_cast<int>(len));
    }
    const int n_tiles = (limit + kKTile - 1) / kKTile;
    const int n_tiles_all = (K + kKTile - 1) / kKTile;
    int tiles_per_block = 1;
    int wrow = 0;  // 32- or 64-row query blocks: this wave's block row in the workgroup
    if constexpr (kBlock) {
        tiles_per_block = static_cast<int>(p.kv_block / kKTile);
        const int words = static_cast<int>((p.n_kv_blocks + 31) / 32);
        const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
        if constexpr (!kMultiRow) {
            for (int i = tid; i < words; i += 256) {
                listed_bits[i] = 0u;
                full_bits[i] = 0u;
            }
            __syncthreads();
            const int64_t list_row = inst * p.n_q_rows + q0 / p.q_block;
            mark_list(listed_bits, p.kv_num_blocks, p.kv_indices, list_row, p.max_blocks,
                      p.n_kv_blocks, tid, 256);
            if (p.full_kv_num_blocks) {
                mark_list(full_bits, p.full_kv_num_blocks, p.full_kv_indices, list_row,
                          p.full_max_blocks, p.n_kv_blocks, tid, 256);
                mark_list(listed_bits, p.full_kv_num_blocks, p.full_kv_indices, list_row,
                          p.full_max_blocks, p.n_kv_blocks, tid, 256);
            }
        } else {
            const int qb = static_cast<int>(p.q_block);
            const int rows = 128 / qb;  // 2 or 4
            wrow = (32 * wave) / qb;
            for (int i = tid; i < (1 + 2 * kRowsMulti) * kMultiWords; i += 256) block_bits[i] = 0u;
            __syncthreads();
            for (int r = 0; r < rows; ++r) {
                const int64_t qrow_blk = q0 / qb + r;
                if (qrow_blk >= p.n_q_rows) break;  // rows past Q
                const int64_t list_row = inst * p.n_q_rows + qrow_blk;
                mark_list(row_listed(r), p.kv_num_blocks, p.kv_indices, list_row, p.max_blocks,
                          p.n_kv_blocks, tid, 256);
                if (p.full_kv_num_blocks) {
                    mark_list(row_full(r), p.full_kv_num_blocks, p.full_kv_indices, list_row,
                              p.full_max_blocks, p.n_kv_blocks, tid, 256);
                    mark_list(row_listed(r), p.full_kv_num_blocks, p.full_kv_indices, list_row,
                              p.full_max_blocks, p.n_kv_blocks, tid, 256);
                }
            }
            __syncthreads();
            for (int i = tid; i < words; i += 256) {
                uint32_t u = 0u;
                for (int r = 0; r < rows; ++r) u |= row_listed(r)[i];
                listed_bits[i] = u;
            }
        }
        __syncthreads();
    }
    auto first_tile = [&]() -> int {
        if constexpr (!kBlock) {
            return n_tiles > 0 ? 0 : -1;
        } else {
            const int64_t blk = next_set(listed_bits, 0, p.n_kv_blocks);
            return blk < 0 ? -1 : static_cast<int>(blk) * tiles_per_block;
        }
    };
    auto next_tile = [&](int t) -> int {
        if (t < 0) return -1;
        if constexpr (!kBlock) {
            return t + 1 < n_tiles ? t + 1 : -1;
        } else {
            if ((t + 1) % tiles_per_block != 0 && t + 1 < n_tiles_all) return t + 1;
            const int64_t blk = next_set(listed_bits, t / tiles_per_block + 1, p.n_kv_blocks);
            return blk < 0 ? -1 : static_cast<int>(blk) * tiles_per_block;
        }
    };

    // ---- this lane's row: Q (B operand), dO (B operand), Delta, -lse log2 e
    // Dn: the head dimension of the data, D that of the tiles (with PAD, Dn <
    // D and a multiple of 8: columns past Dn enter as zeros and are not stored)
    const int Dn = PAD ? static_cast<int>(p.D) : D;
    v8 qop[D / 16], gop[D / 16];
    float delta = 0.f;
    {
        const int64_t roff = (bnh * p.Q + qload) * Dn;
        const T* qp = static_cast<const T*>(p.q) + roff;
        const T* gp = static_cast<const T*>(g.dout) + roff;
        const T* op = static_cast<const T*>(g.out) + roff;
        float part = 0.f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int c0 = 16 * st + 8 * half;
            v8 x = load8_or_zero<v8>(qp, c0, Dn);
            if (EXACT) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = static_cast<T>(static_cast<float>(x[j]) * p.scale);
            }
            qop[st] = x;
            gop[st] = load8_or_zero<v8>(gp, c0, Dn);
            const v8 o = load8_or_zero<v8>(op, c0, Dn);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                part = fmaf(static_cast<float>(gop[st][j]), static_cast<float>(o[j]), part);
        }
        delta = sum_halves(part);
    }
    const int64_t ridx = bnh * p.Q + qload;
    const bool live = row_ok && g.mx[ridx] != kMaskedLogit;
    const float nl2 = live ? -g.lse[ridx] * kLog2e : -INFINITY;
    const float c_exp = (EXACT ? 1.0f : p.scale) * kLog2e;
    const float inv_s = EXACT ? 1.0f : 1.0f / p.scale;

    // ---- DMA ----------------------------------------------------------------
    const uint32_t kv_bytes = static_cast<uint32_t>(p.K * Dn * sizeof(T));
    const u32x4 k_desc = make_desc(static_cast<const T*>(p.k) + bnh * p.K * Dn, kv_bytes);
    const u32x4 v_desc = make_desc(static_cast<const T*>(p.v) + bnh * p.K * Dn, kv_bytes);
    const uint32_t mem_tile = static_cast<uint32_t>(32 * 2 * Dn);  // one tile of rows in memory
    auto kbuf = [&](int x) { return (lds_char*)(x == 0 ? k_lds0 : x == 1 ? k_lds1 : k_lds2); };
    auto vbuf = [&](int x) { return (lds_char*)(x == 0 ? v_lds0 : x == 1 ? v_lds1 : v_lds2); };
    uint32_t kv_src[kKvDma];
#pragma unroll
    for (int j = 0; j < kKvDma; ++j) kv_src[j] = Ge::dma_src((wave + 4 * j) % Ge::tileDma, lane, Dn);
    auto dma_kv = [&](int t, int x) {
        const uint32_t toff = t >= 0 ? static_cast<uint32_t>(t) * mem_tile : kNoTile;
#pragma unroll
        for (int j = 0; j < kKvDma; ++j) {
            const int I = wave + 4 * j;
            if (I < Ge::tileDma)
                dma16(k_desc, kbuf(x) + 1024 * I, kv_src[j] + toff);
            else
                dma16(v_desc, vbuf(x) + 1024 * (I - Ge::tileDma), kv_src[j] + toff);
        }
    };
    // bias block (the forward kernel's layout): instruction j, lane l fills
    // row r = 8 j + l / 8, stored chunk l % 8, from source chunk (l % 8) ^ fb(r)
    const char* bplane = BIAS != kBNone ? reinterpret_cast<const char*>(p.bias + (b * p.H + h) * p.Q * p.K) : nullptr;
    const uint32_t bias_bytes = BIAS != kBNone ? static_cast<uint32_t>(p.Q * p.K * 4) : 0u;
    const u32x4 b_desc = make_desc(bplane, bias_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(bplane, bias_bytes);
    lds_char* const bias_lds = (lds_char*)b_lds + (BIAS == kBLds ? wave * kBiasWaveBytes : 0);
    const uint32_t b_row = static_cast<uint32_t>(q0w + (lane >> 3)) * static_cast<uint32_t>(K) * 4u;
    const uint32_t b_src_even = b_row + 16u * static_cast<uint32_t>((lane & 7) ^ (lane >> 4));
    const uint32_t b_src_odd = b_row + 16u * static_cast<uint32_t>((lane & 7) ^ (lane >> 4) ^ 4);
    auto dma_bias = [&](int t) {
        if constexpr (BIAS == kBLds) {
            const uint32_t toff = static_cast<uint32_t>(t) * kBiasRowBytes;
#pragma unroll
            for (int j = 0; j < kBiasDma; ++j) {
                const uint32_t rws = static_cast<uint32_t>(8 * j) * static_cast<uint32_t>(K) * 4u;
                dma16(b_desc, bias_lds + 1024 * j, ((j & 1) ? b_src_odd : b_src_even) + rws + toff);
            }
        }
    };
    const uint32_t bias_lane = static_cast<uint32_t>(qload) * static_cast<uint32_t>(K) * 4u + 16u * half;

    // Dense key mask as bits (the forward kernel's scheme): lane i of
    // dense_word holds the validity of the 32 keys of tile 64 c + i.
    const uint8_t* dense_row = kDense ? p.dense + (b * p.N + n) * p.K : nullptr;
    uint32_t dense_word = 0;
    int dense_chunk = -1;
    auto load_dense_chunk = [&](int c) {
        const int t0 = 64 * c;
        const int nt = min(64, n_tiles_all - t0);
        uint32_t w = 0;
        for (int i0 = 0; i0 < nt; i0 += 16) {
            bool v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = (t0 + i0 + 2 * j) * kKTile + lane;
                v[j] = kk < K && dense_row[kk] != 0;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint64_t bits = __ballot(v[j]);
                w = lane == i0 + 2 * j ? static_cast<uint32_t>(bits) : w;
                w = lane == i0 + 2 * j + 1 ? static_cast<uint32_t>(bits >> 32) : w;
            }
        }
        dense_word = w;
        dense_chunk = c;
    };

    const int rrd = Ge::row_base(col, half);
    const int tr0 = Ge::tr_base(lane, 0), tr1 = Ge::tr_base(lane, 1);
    // bias read into the accumulator layout: register 4 g + e is key 8 g +
    // 4 half + e, source chunk 2 g + half of row col
    int b_rd[4];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) b_rd[gg] = col * kBiasRowBytes + 16 * ((2 * gg + half) ^ fb(col));

    f32x16 acc[D / 32];
#pragma unroll
    for (int jb = 0; jb < D / 32; ++jb) acc[jb] = f32x16{};

    auto compute = [&](int t, int x, auto dma) {
        const int k0 = t * kKTile;
        const lds_char* kt = kbuf(x);
        const lds_char* vt = vbuf(x);
        f32x16 z, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = -delta;
        if constexpr (BIAS == kBLds) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const f32x4 bv = __builtin_bit_cast(f32x4, *reinterpret_cast<const lds_u32x4*>(bias_lds + b_rd[gg]));
#pragma unroll
                for (int e = 0; e < 4; ++e) z[4 * gg + e] = bv[e];
            }
        } else if constexpr (BIAS == kBScalar) {
            const uint32_t base = bias_lane + static_cast<uint32_t>(k0) * 4u;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg)
#pragma unroll
                for (int e = 0; e < 4; ++e) z[4 * gg + e] = bload32(b_rsrc, base + 4u * (8 * gg + e));
        } else {
            z = f32x16{};
        }
        if (BIAS != kBNone && !EXACT) z *= inv_s;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) z = M::run(row_operand<v8>(kt, rrd, st), qop[st], z);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) dp = M::run(row_operand<v8>(vt, rrd, st), gop[st], dp);
        dma();
        // ---- element mask (only on tiles that need one) --------------------
        bool need_mask = k0 + kKTile > limit;
        bool causal = false;
        uint32_t dense_bits = ~0u;
        if constexpr (kDense) {
            if ((t >> 6) != dense_chunk) load_dense_chunk(t >> 6);
            dense_bits = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dense_word), t & 63));
            need_mask = need_mask || dense_bits != ~0u;
        }
        bool unlisted = false;  // a tile visited for another block row of the workgroup
        if constexpr (kBlock) {
            const int blk = t / tiles_per_block;
            if (kMultiRow && !bit_set(row_listed(wrow), blk)) {
                unlisted = true;
                need_mask = true;
            } else if (p.mask_mod == TRIATTN_MOD_CAUSAL &&
                       !bit_set(kMultiRow ? row_full(wrow) : full_bits, blk) && k0 + kKTile - 1 > q0w) {
                causal = true;
                need_mask = true;
            }
        }
        if (need_mask) {
            const int room = limit - k0;
            uint32_t w = room >= kKTile ? ~0u : room <= 0 ? 0u : (1u << room) - 1u;
            if (kDense) w &= dense_bits;
            if constexpr (kMultiRow) {
                if (unlisted) w = 0u;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ka = 8 * (r / 4) + (r % 4);
                const uint32_t lo = static_cast<uint32_t>(static_cast<int32_t>(w << (31 - ka)) >> 31);
                const uint32_t hi = static_cast<uint32_t>(static_cast<int32_t>(w << (27 - ka)) >> 31);
                bool ok = __builtin_amdgcn_inverse_ballot_w64(lo | (static_cast<uint64_t>(hi) << 32));
                if (causal) ok = ok && qrow >= k0 + ka + 4 * half;
                z[r] = ok ? z[r] : -INFINITY;
            }
        }
        v8 dzop[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(z[r], c_exp, nl2));
            dzop[r / 8][r % 8] = static_cast<T>(pr * dp[r]);
        }
#pragma unroll
        for (int jb = 0; jb < D / 32; ++jb)
#pragma unroll
            for (int st = 0; st < 2; ++st)
                acc[jb] = M::run(tr_operand<v8, D>(kt, tr0, tr1, jb, st), dzop[st], acc[jb]);
    };

    // ---- key-tile loop: ring position j holds tile t_j in buffers j % 3 ----
    int cur = first_tile();
    int nxt = next_tile(cur);
    if (cur >= 0) {
        if constexpr (kDense) load_dense_chunk(cur >> 6);  // before any DMA is in flight
        dma_bias(cur);
        dma_kv(cur, 0);
        dma_kv(nxt, 1);
        wait_vmem();
        __syncthreads();
    }
    auto step = [&](auto X) {
        constexpr int x = decltype(X)::value;
        const int nxt2 = __builtin_amdgcn_readfirstlane(next_tile(nxt));
        __builtin_amdgcn_s_waitcnt(kVmcntWait<kKvDma>());
        __syncthreads();
        compute(cur, x, [&] {
            if (nxt >= 0) {
                wait_lds();
                dma_bias(nxt);
            }
            dma_kv(nxt2, (x + 2) % 3);
        });
        cur = nxt;
        nxt = nxt2;
    };
    while (cur >= 0) {
        step(Par<0>{});
        if (cur < 0) break;
        step(Par<1>{});
        if (cur < 0) break;
        step(Par<2>{});
    }
    wait_vmem();

    if (!row_ok) return;
    T* dqr = static_cast<T*>(g.dq) + (bnh * p.Q + qrow) * Dn;
#pragma unroll
    for (int jb = 0; jb < D / 32; ++jb)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (32 * jb + 8 * c + 4 * half < Dn)  // (not a padding column)
                store4(dqr + 32 * jb + 8 * c + 4 * half, acc[jb][4 * c] * p.scale, acc[jb][4 * c + 1] * p.scale,
                   acc[jb][4 * c + 2] * p.scale, acc[jb][4 * c + 3] * p.scale);
}

// ---- dBias ---------------------------------------------------------------
// dB_qk = sum over n, in order, of dz_qk.  One workgroup of QW x KW waves per
// (b, h, 32 QW query rows, 32 KW keys, range of n); wave w takes rows
// 32 (w % QW) .. + 31 and keys 32 (w / QW) .. + 31 in the dQ kernel's layout
// (lane l: row 32 (w % QW) + l % 32, 16 keys in registers), and keeps its
// 32 x 32 bias block (divided by s) as the C operand and its sums in
// registers.  Per n, the workgroup's rows of Q and dO, its keys of K and V and
// the row data arrive by LDS DMA, `slots - 1` n ahead in a ring:
//   z^T = K Q^T + C,  dP^T = V dO^T - Delta   A = K, V rows, B = Q, dO rows
// (-Delta is the initial accumulator of dP^T), P = exp2(z c - lse log2 e),
// dB += P dP^T.  n whose length leaves no key of the workgroup valid are
// skipped; the ragged tile and the dense mask select per element; rows with
// no valid key contribute nothing.  With more than one range of n (splits),
// each range's sums go to its own plane of the workspace and
// bwd_dbias_combine_kernel adds the planes in range order.
template <int D>
struct DbGeo {
    static constexpr int QW = D <= 64 ? 4 : 2;  // waves along the query rows
    static constexpr int KW = D <= 64 ? 4 : 2;  // waves along the keys
    static constexpr int waves = QW * KW;
    static constexpr int slots = 2;
    static constexpr int rowsQ = 32 * QW, rowsK = 32 * KW;
    static constexpr int tileBytes = BGeo<D>::tileBytes;
    // one n: QW tiles of Q, QW of dO, KW of K, KW of V
    static constexpr int slotBytes = (2 * QW + 2 * KW) * tileBytes;
    static constexpr int dmaPerWave = slotBytes / 1024 / waves;
    static_assert(dmaPerWave * waves * 1024 == slotBytes, "DMAs split evenly over the waves");
    static constexpr int infoBytes = rowsQ * 8;  // row data (QW tiles of 256 bytes)
    static constexpr int infoWaves = infoBytes / 128;  // waves issuing an 8-lane row-data DMA
    static_assert(infoWaves >= 1 && infoWaves <= waves, "row data in 128-byte pieces");
    static constexpr int keyWords = rowsK / 64;  // 64-bit validity words per n
};

template <typename T, int D, int KIND, bool PAD>
__global__ __launch_bounds__(64 * DbGeo<D>::waves) void bwd_dbias_kernel(Params p, BwdParams g,
                                                                        const float* rows,
                                                                        float* part, int splits) {
    using M = Mma<T>;
    using v8 = typename M::v8;
    using Ge = BGeo<D>;
    using G = DbGeo<D>;
    constexpr bool kDense = KIND == TRIATTN_MASK_DENSE;
    constexpr bool kLens = KIND == TRIATTN_MASK_KV_LENGTHS;
    constexpr bool kBlockM = KIND == TRIATTN_MASK_BLOCK;
    constexpr int R = G::slots;
    static_assert(R == 2, "every position waits for all DMAs (counts differ between waves)");
    __shared__ __attribute__((aligned(1024))) char t_lds[R][G::slotBytes];
    __shared__ __attribute__((aligned(1024))) char r_lds[R][G::infoBytes];
    // Bit i of valid_w[(m - c0) keyWords + i / 64]: key k0 + i valid for n =
    // m, for a chunk of n
    // starting at c0.  Built before the ring starts, so that the loop issues
    // no memory load besides the DMAs (a wait for such a load would also wait
    // for the DMAs issued before it).
    constexpr int kChunkN = 512;
    __shared__ uint64_t valid_w[kChunkN * G::keyWords];
    // Block lists (query blocks of 32, 64 or a multiple of 128 rows, kv
    // blocks of whole 32-key tiles: each wave's 32 x 32 block lies in one
    // block row and one kv block): per n of the chunk, bits 2w and 2w + 1 of
    // blk_w say whether wave w's kv block is listed (kv or full list) and full.
    static_assert(G::waves <= 16, "two bits per wave in a word");
    __shared__ uint32_t blk_w[kBlockM ? kChunkN : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int qg = wave % G::QW, kg = wave / G::QW;

    // ---- workgroup -> (b, h, range of n, query tile, key tile), XCD-contiguous
    const int64_t n_qt = (p.Q + G::rowsQ - 1) / G::rowsQ, n_kt = (p.K + G::rowsK - 1) / G::rowsK;
    const int64_t lid = xcd_order(blockIdx.x, gridDim.x);
    const int64_t kt = lid % n_kt;
    const int64_t qt = (lid / n_kt) % n_qt;
    const int64_t sp = (lid / (n_kt * n_qt)) % splits;
    const int64_t h = (lid / (n_kt * n_qt * splits)) % p.H;
    const int64_t b = lid / (n_kt * n_qt * splits * p.H);
    const int K = static_cast<int>(p.K), Q = static_cast<int>(p.Q), N = static_cast<int>(p.N);
    const int q0 = static_cast<int>(qt) * G::rowsQ, k0 = static_cast<int>(kt) * G::rowsK;
    const int n_begin = static_cast<int>(sp * N / splits), n_end = static_cast<int>((sp + 1) * N / splits);
    const int qrow = q0 + 32 * qg + col;  // this lane's query
    const int kw = k0 + 32 * kg;          // this wave's first key
    const int64_t n_t32 = (p.Q + 31) / 32;  // 32-row tiles of the row data per slice

    // scale: z = s (Q.K + B / s); s = 0 leaves z = B
    const bool zero_s = p.scale == 0.0f;
    const float s_eff = zero_s ? 1.0f : p.scale;
    const float c_exp = s_eff * kLog2e, inv_s = 1.0f / s_eff;

    // bias block in the accumulator layout: register 4 g + e is key kw + 8 g + 4 half + e
    const char* bplane = reinterpret_cast<const char*>(p.bias + (b * p.H + h) * p.Q * p.K);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(bplane, static_cast<uint32_t>(p.Q * p.K * 4));
    f32x16 cb;
    {
        const uint32_t base = (static_cast<uint32_t>(qrow) * static_cast<uint32_t>(K) + kw) * 4u + 16u * half;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
#pragma unroll
            for (int e = 0; e < 4; ++e) cb[4 * gg + e] = bload32(b_rsrc, base + 4u * (8 * gg + e)) * inv_s;
    }

    // key validity words of n = c0 .. c1 - 1 (the workgroup's rowsK keys)
    int c0 = n_begin, c1 = n_begin;
    auto fill_valid = [&]() {
        for (int i = tid; i < (c1 - c0) * G::keyWords; i += 64 * G::waves) {
            const int m = c0 + i / G::keyWords;
            const int kb = k0 + 64 * (i % G::keyWords);  // first key of the word
            uint64_t word = ~0ull;
            if constexpr (kLens) {
                if (p.kv_lengths) {
                    const int64_t len = p.kv_lengths[b * p.N + m];
                    const int lim = len < 0 ? 0 : (len > K ? K : static_cast<int>(len));
                    const int rel = lim - kb;
                    word = rel >= 64 ? ~0ull : rel <= 0 ? 0ull : (1ull << rel) - 1ull;
                }
            } else if constexpr (kDense) {
                const uint8_t* drow = p.dense + (b * p.N + m) * p.K;
                word = 0ull;
                for (int j = 0; j < 64 && kb + j < K; ++j)
                    if (drow[kb + j] != 0) word |= 1ull << j;
            }
            valid_w[i] = word;
        }
        if constexpr (kBlockM) {
            for (int i = tid; i < c1 - c0; i += 64 * G::waves) blk_w[i] = 0u;
            __syncthreads();
            // one thread per (n, query sub-tile, list entry)
            const int64_t inst0 = b * p.stride_b + h * p.stride_h;
            const int64_t wl = p.max_blocks, wf = p.full_kv_num_blocks ? p.full_max_blocks : 0;
            const int64_t per = G::QW * (wl + wf);
            const int64_t total = static_cast<int64_t>(c1 - c0) * per;
            for (int64_t e = tid; e < total; e += 64 * G::waves) {
                const int m = c0 + static_cast<int>(e / per);
                const int64_t r = e % per;
                const int qgi = static_cast<int>(r / (wl + wf));
                const int64_t j = r % (wl + wf);
                const int qs = q0 + 32 * qgi;  // the sub-tile's first query
                if (qs >= Q) continue;
                const int64_t row = (inst0 + m * p.stride_n) * p.n_q_rows + qs / p.q_block;
                const bool full = j >= wl;
                const int32_t* counts = full ? p.full_kv_num_blocks : p.kv_num_blocks;
                const int32_t* ids = full ? p.full_kv_indices : p.kv_indices;
                const int64_t width = full ? wf : wl, jj = full ? j - wl : j;
                int64_t cnt = counts[row];
                cnt = cnt < 0 ? 0 : (cnt > width ? width : cnt);
                if (jj >= cnt) continue;
                const int64_t id = ids[row * width + jj];
                uint32_t bits = 0u;
#pragma unroll
                for (int kgi = 0; kgi < G::KW; ++kgi) {
                    const int ks = k0 + 32 * kgi;  // the sub-tile's first key
                    if (ks < K && id == ks / p.kv_block) bits |= (full ? 3u : 1u) << (2 * (qgi + G::QW * kgi));
                }
                if (bits) atomicOr(&blk_w[m - c0], bits);
            }
        }
    };
    auto any_valid = [&](int m) {
        bool any = false;
#pragma unroll
        for (int j = 0; j < G::keyWords; ++j) any = any || valid_w[(m - c0) * G::keyWords + j] != 0ull;
        return any;
    };
    // first n >= m0 of the chunk with a valid key, or -1
    auto next_n = [&](int m0) -> int {
        if (m0 < 0) return -1;
        if constexpr (!kLens && !kDense) {
            return m0 < c1 ? m0 : -1;
        } else {
            for (int base = m0; base < c1; base += 64) {
                const int m = base + lane;
                const uint64_t bits = __ballot(m < c1 && any_valid(m));
                if (bits) return base + static_cast<int>(__builtin_ctzll(bits));
            }
            return -1;
        }
    };

    // DMA of one n: instruction I = wave + waves j; tile I / tileDma of the
    // slot (Q tiles, dO tiles, K tiles, V tiles), piece I % tileDma
    // (rows of Dn elements in memory; with PAD the columns past Dn are zeros)
    const int Dn = PAD ? static_cast<int>(p.D) : D;
    const uint32_t mem_row = static_cast<uint32_t>(2 * Dn);
    uint32_t src[G::dmaPerWave];
#pragma unroll
    for (int j = 0; j < G::dmaPerWave; ++j) src[j] = Ge::dma_src((wave + G::waves * j) % Ge::tileDma, lane, Dn);
    const uint32_t qbytes = static_cast<uint32_t>(p.Q * Dn * sizeof(T));
    const uint32_t kbytes = static_cast<uint32_t>(p.K * Dn * sizeof(T));
    auto dma_n = [&](int m, int x) {
        const int64_t bnh = (b * p.N + (m >= 0 ? m : 0)) * p.H + h;
        const u32x4 dq = make_desc(static_cast<const T*>(p.q) + bnh * p.Q * Dn, qbytes);
        const u32x4 dg = make_desc(static_cast<const T*>(g.dout) + bnh * p.Q * Dn, qbytes);
        const u32x4 dk = make_desc(static_cast<const T*>(p.k) + bnh * p.K * Dn, kbytes);
        const u32x4 dv = make_desc(static_cast<const T*>(p.v) + bnh * p.K * Dn, kbytes);
        const u32x4 dr = make_desc(rows + bnh * n_t32 * 64, static_cast<uint32_t>(n_t32 * 256));
#pragma unroll
        for (int j = 0; j < G::dmaPerWave; ++j) {
            const int I = wave + G::waves * j;
            const int tile = I / Ge::tileDma;
            lds_char* dst = (lds_char*)t_lds[x] + 1024 * I;
            if (tile < G::QW) {
                const uint32_t o = static_cast<uint32_t>(q0 + 32 * tile) * mem_row + src[j];
                dma16(dq, dst, m >= 0 ? o : kNoTile);
            } else if (tile < 2 * G::QW) {
                const uint32_t o = static_cast<uint32_t>(q0 + 32 * (tile - G::QW)) * mem_row + src[j];
                dma16(dg, dst, m >= 0 ? o : kNoTile);
            } else if (tile < 2 * G::QW + G::KW) {
                // (s = 0: the K tiles are zeros, so Q.K adds exactly 0 to B)
                const uint32_t o = static_cast<uint32_t>(k0 + 32 * (tile - 2 * G::QW)) * mem_row + src[j];
                dma16(dk, dst, m >= 0 && !zero_s ? o : kNoTile);
            } else {
                const uint32_t o = static_cast<uint32_t>(k0 + 32 * (tile - 2 * G::QW - G::KW)) * mem_row + src[j];
                dma16(dv, dst, m >= 0 ? o : kNoTile);
            }
        }
        // 128 bytes per wave of the row data of tiles q0 / 32 ..
        if (wave < G::infoWaves) {
            const uint32_t roff = m >= 0 ? static_cast<uint32_t>((q0 / 32) * 256 + 128 * wave + 16 * lane) : kNoTile;
            if (lane < 8) dma16(dr, (lds_char*)r_lds[x] + 128 * wave, roff);
        }
    };

    const int rrd = Ge::row_base(col, half);
    const int q_tile = qg * Ge::tileBytes, g_tile = (G::QW + qg) * Ge::tileBytes;
    const int k_tile = (2 * G::QW + kg) * Ge::tileBytes, v_tile = (2 * G::QW + G::KW + kg) * Ge::tileBytes;

    f32x16 acc{};
    auto compute = [&](int m, int x) {
        const lds_char* t = (const lds_char*)t_lds[x];
        const lds_char* ri = (const lds_char*)r_lds[x] + 256 * qg + 4 * col;  // tile qg, row col
        const float ndelta = *reinterpret_cast<const __attribute__((address_space(3))) float*>(ri);
        float nl2 = *reinterpret_cast<const __attribute__((address_space(3))) float*>(ri + 128);
        nl2 = nl2 != nl2 ? -INFINITY : nl2;  // no valid key: no contribution
        // (no branch on s = 0 here: a phi of z would copy the bias block
        // into the MFMA's registers on every n)
        f32x16 z = cb, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = ndelta;
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            z = M::run(row_operand<v8>(t + k_tile, rrd, st), row_operand<v8>(t + q_tile, rrd, st), z);
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            dp = M::run(row_operand<v8>(t + v_tile, rrd, st), row_operand<v8>(t + g_tile, rrd, st), dp);
        // keys valid for this n (the ragged tile of a length, the dense mask)
        uint32_t w = static_cast<uint32_t>(valid_w[(m - c0) * G::keyWords + kg / 2] >> (32 * (kg % 2)));
        bool causal = false;  // block lists: the causal mask_mod on a listed, not full block
        if constexpr (kBlockM) {
            const uint32_t st = (blk_w[m - c0] >> (2 * wave)) & 3u;
            if (st == 0u)
                w = 0u;
            else if (st == 1u && p.mask_mod == TRIATTN_MOD_CAUSAL && kw + 31 > q0 + 32 * qg)
                causal = true;
        }
        if (w != ~0u || causal) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ka = 8 * (r / 4) + (r % 4);
                const uint32_t lo = static_cast<uint32_t>(static_cast<int32_t>(w << (31 - ka)) >> 31);
                const uint32_t hi = static_cast<uint32_t>(static_cast<int32_t>(w << (27 - ka)) >> 31);
                bool ok = __builtin_amdgcn_inverse_ballot_w64(lo | (static_cast<uint64_t>(hi) << 32));
                if constexpr (kBlockM) ok = ok && (!causal || qrow >= kw + ka + 4 * half);
                z[r] = ok ? z[r] : -INFINITY;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = fmaf(__builtin_amdgcn_exp2f(fmaf(z[r], c_exp, nl2)), dp[r], acc[r]);
    };

    // chunks of the range; in each, ring position j holds n_j in slot j % R,
    // loaded R - 1 positions ahead
    for (c0 = n_begin; c0 < n_end; c0 = c1) {
        c1 = min(c0 + kChunkN, n_end);
        __syncthreads();  // the previous chunk's words are no longer read
        fill_valid();
        __syncthreads();
        int ns[R];
        ns[0] = next_n(c0);
#pragma unroll
        for (int i = 1; i < R; ++i) ns[i] = next_n(ns[i - 1] >= 0 ? ns[i - 1] + 1 : -1);
        if (ns[0] < 0) continue;
#pragma unroll
        for (int i = 0; i < R - 1; ++i) dma_n(ns[i], i);
        int x = 0;
        while (ns[0] >= 0) {
            // every DMA has landed (the ring of two is loaded one n ahead)
            wait_vmem();
            __syncthreads();  // slot x landed for every wave; slot x - 1 is free
            dma_n(ns[R - 1], (x + R - 1) % R);
            compute(ns[0], x);
#pragma unroll
            for (int i = 0; i < R - 1; ++i) ns[i] = ns[i + 1];
            ns[R - 1] = next_n(ns[R - 2] >= 0 ? ns[R - 2] + 1 : -1);
            x = (x + 1) % R;
        }
        wait_vmem();
    }

    if (qrow >= Q) return;
    float* dst = (splits > 1 ? part + sp * p.B * p.H * p.Q * p.K : g.dbias) + ((b * p.H + h) * p.Q + qrow) * p.K;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kk = kw + 8 * (r / 4) + 4 * half + (r % 4);
        if (kk < K) dst[kk] = acc[r];
    }
}

// dBias = the sum of the splits' planes, in split order.  Four elements per
// thread (16-byte loads of every plane issued together) when the plane size
// and the pointers allow it; the tail and other shapes one at a time.
constexpr int kMaxSplits = 8;
__global__ __launch_bounds__(256) void bwd_dbias_combine_kernel(float* dbias, const float* part,
                                                                int64_t count, int splits) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    const bool vec = splits <= kMaxSplits && count % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(dbias) % 16 == 0;
    const int64_t n4 = vec ? count / 4 : 0;
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        f32x4 v[kMaxSplits];
#pragma unroll
        for (int j = 0; j < kMaxSplits; ++j)
            if (j < splits) v[j] = reinterpret_cast<const f32x4*>(part + j * count)[i];
        f32x4 s = v[0];
#pragma unroll
        for (int j = 1; j < kMaxSplits; ++j)
            if (j < splits) s += v[j];
        reinterpret_cast<f32x4*>(dbias)[i] = s;
    }
    for (int64_t i = 4 * n4 + blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
        float s = part[i];
        for (int j = 1; j < splits; ++j) s += part[j * count + i];
        dbias[i] = s;
    }
}

// ---- launch -----------------------------------------------------------------
// The workspace holds the row data: 8 B N H Q bytes of (Delta, -lse log2 e)
// pairs, then one uint32 per 32-row tile.
template <typename T, int D, int KIND, int BIAS, bool EXACT, bool PAD>
void launch_bwd_pair(const Params& p, const BwdParams& g, float* rows, uint32_t* tdead, dim3 gdk,
                     dim3 gdq, hipStream_t stream) {
    const dim3 block(256);
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, KIND, BIAS, EXACT, PAD>), gdk, block, 0, stream, p, g, rows, tdead);
    if constexpr (KIND == TRIATTN_MASK_BLOCK) {
        if (p.q_block < 128) {  // 32- or 64-row query blocks
            hipLaunchKernelGGL((bwd_dq_kernel<T, D, kBwdBlockRows, BIAS, EXACT, PAD>), gdq, block, 0, stream,
                               p, g);
            return;
        }
    }
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, KIND, BIAS, EXACT, PAD>), gdq, block, 0, stream, p, g);
}

template <typename T, int D, int KIND, int BIAS>
hipError_t launch_bwd_bias(const Params& p, const BwdParams& g, bool exact, float* rows,
                           uint32_t* tdead, hipStream_t stream) {
    const int64_t bnh = p.B * p.N * p.H;
    const int64_t gk = bnh * ((p.K + 127) / 128), gq = bnh * ((p.Q + 127) / 128);
    if (gk > 0x7fffffff || gq > 0x7fffffff) return hipErrorInvalidConfiguration;
    // head dimensions between the tile widths take the padded instantiations
    const dim3 gdk(static_cast<unsigned>(gk)), gdq(static_cast<unsigned>(gq));
    const bool pad = p.D != D;
    if (exact && !pad)
        launch_bwd_pair<T, D, KIND, BIAS, true, false>(p, g, rows, tdead, gdk, gdq, stream);
    else if (!pad)
        launch_bwd_pair<T, D, KIND, BIAS, false, false>(p, g, rows, tdead, gdk, gdq, stream);
    else if (exact)
        launch_bwd_pair<T, D, KIND, BIAS, true, true>(p, g, rows, tdead, gdk, gdq, stream);
    else
        launch_bwd_pair<T, D, KIND, BIAS, false, true>(p, g, rows, tdead, gdk, gdq, stream);
    return hipGetLastError();
}

template <typename T, int D, int KIND>
hipError_t launch_bwd_kind(const Params& p, const BwdParams& g, bool exact, float* ws,
                           size_t ws_bytes, hipStream_t stream) {
    const int64_t tiles = p.B * p.N * p.H * ((p.Q + 31) / 32);
    float* rows = ws;
    uint32_t* tdead = reinterpret_cast<uint32_t*>(ws + 64 * tiles);
    const unsigned gr = static_cast<unsigned>(tiles < (1 << 20) ? tiles : (1 << 20));
    if (p.D != D)
        hipLaunchKernelGGL((bwd_rows_kernel<T, D, true>), dim3(gr), dim3(4 * D), 0, stream, p, g, rows, tdead);
    else
        hipLaunchKernelGGL((bwd_rows_kernel<T, D, false>), dim3(gr), dim3(4 * D), 0, stream, p, g, rows, tdead);
    hipError_t e;
    if (!p.bias)
        e = launch_bwd_bias<T, D, KIND, kBNone>(p, g, exact, rows, tdead, stream);
    else if (p.K % 4 == 0 && reinterpret_cast<uintptr_t>(p.bias) % 16 == 0)
        e = launch_bwd_bias<T, D, KIND, kBLds>(p, g, exact, rows, tdead, stream);
    else
        e = launch_bwd_bias<T, D, KIND, kBScalar>(p, g, exact, rows, tdead, stream);
    if (e != hipSuccess) return e;
    {
        if (g.dbias && p.bias) {
            using G = DbGeo<D>;
            // splits beyond the first need a plane of partial sums each, after
            // the row data
            const int64_t plane = p.B * p.H * p.Q * p.K;
            const size_t used = static_cast<size_t>(bwd_rows_bytes(p.B * p.N * p.H, p.Q));
            const size_t room = ws_bytes > used ? ws_bytes - used : 0;
            int splits = dbias_splits(p.B, p.N, p.H, p.Q, p.K, D);
            while (splits > 1 && room < static_cast<size_t>(4 * splits * plane)) --splits;
            float* part = ws + used / 4;
            const int64_t gb = p.B * p.H * ((p.Q + G::rowsQ - 1) / G::rowsQ) *
                               ((p.K + G::rowsK - 1) / G::rowsK) * splits;
            if (gb > 0x7fffffff) return hipErrorInvalidConfiguration;
            if (p.D != D)
                hipLaunchKernelGGL((bwd_dbias_kernel<T, D, KIND, true>), dim3(static_cast<unsigned>(gb)),
                                   dim3(64 * G::waves), 0, stream, p, g, rows, part, splits);
            else
                hipLaunchKernelGGL((bwd_dbias_kernel<T, D, KIND, false>), dim3(static_cast<unsigned>(gb)),
                                   dim3(64 * G::waves), 0, stream, p, g, rows, part, splits);
            static_assert(kMaxSplits >= 8, "dbias_splits returns at most 8");
            if (splits > 1) {
                const int64_t want = (plane / 4 + 255) / 256 + 1;
                const unsigned gc = static_cast<unsigned>(want < 8192 ? want : 8192);
                hipLaunchKernelGGL(bwd_dbias_combine_kernel, dim3(gc), dim3(256), 0, stream,
                                   g.dbias, part, plane, splits);
            }
        }
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_d(const Params& p, const BwdParams& g, bool exact, float* ws,
                        size_t ws_bytes, hipStream_t stream) {
    switch (p.mask_kind) {
    case TRIATTN_MASK_NONE:
    case TRIATTN_MASK_KV_LENGTHS:
        return launch_bwd_kind<T, D, TRIATTN_MASK_KV_LENGTHS>(p, g, exact, ws, ws_bytes, stream);
    case TRIATTN_MASK_DENSE:
        return launch_bwd_kind<T, D, TRIATTN_MASK_DENSE>(p, g, exact, ws, ws_bytes, stream);
    case TRIATTN_MASK_BLOCK:
        return launch_bwd_kind<T, D, TRIATTN_MASK_BLOCK>(p, g, exact, ws, ws_bytes, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace triattn
