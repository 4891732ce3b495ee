// MFMA forward kernel for bf16 / fp16 inputs: tiles of width D in {32, 64,
// 128, 256}, serving every head dimension that is a multiple of 8 up to 256
// (those between the widths through the PAD instantiations, zero columns).
//
// Computes the triangle_attention page's equation: per (b, n, h) row,
// O_q = sum_k softmax_k(s Q_q.K_k + B_qk, masked keys excluded) V_k, with the
// lse / max auxiliaries, as a single pass over key tiles (an online,
// max-shifted softmax; the page fixes the result, not the schedule).
//
// Work decomposition: one workgroup of 4 wavefronts owns 128 query rows of
// one (b, n, h); wave w owns rows 32w .. 32w+31.  Keys go in tiles of 32,
// which keeps the LDS footprint (and register state) small enough for four
// workgroups per CU.
//
// Both contractions run on v_mfma_f32_32x32x16_{bf16,f16}:
//   S^T = K . Q^T + C   A = K rows from LDS (16-byte reads), B = Q^T held in
//                   registers for the whole key loop.  The accumulator puts
//                   one query per lane and 16 keys per lane in registers, so
//                   the softmax row reductions are in-lane plus one
//                   v_permlane32_swap with the partner lane (lane ^ 32).
//                   C is the fp32 bias tile itself, so the bias add costs no
//                   vector instruction.
//   O^T = V^T . P^T B = P^T taken directly from the S^T registers (converted
//                   to bf16/fp16), A = V^T read from the row-major V tile with
//                   ds_read_b64_tr_b16, which hands each lane four keys of
//                   one column.  The query stays in the lane, so the running
//                   rescale of O is a per-lane scalar.
//
// Data movement: every tile arrives by LDS DMA (buffer_load ... lds), never
// through registers.  K and V tiles are shared by the workgroup in rings of
// three buffers, loaded two tiles ahead.  The fp32 bias is the largest
// stream (it is re-read for every n):
// the accumulator layout would make each lane fetch 16 bytes from its own
// query row, 32 rows per instruction, which saturates the L1 address path.
// Instead each wave DMAs its 32 x 32 bias block with whole rows per lane
// group (8 cache lines per instruction) into its own LDS region, reads it
// back in the accumulator layout, and immediately refills the region with
// the next tile's block.  LDS rows are unpadded; 16-byte chunks are stored
// XOR-swizzled by row so that the operand reads are bank-conflict free.
//
// Buffer descriptors bound every access to its (b, n, h) slice.  The range
// check covers the per-lane offset (not the scalar one), so no variable
// offset goes in the scalar one: a tile's offset moves the descriptor's base
// (its size shrinking by as much, to 0 for a missing tile) and the rest is
// per lane.  Reads past a slice return 0 and touch no memory, and ragged
// tiles need no clamping (those keys are masked).
//
// Scale: z = s*(Q.K) + B.  When s is 0 or a power of two, s*Q is exact in the
// input format, so Q is scaled once at load and S = (sQ).K + B is z itself.
// Otherwise C holds B/s and z = s*S.  Either way the exponent is one FMA:
// p = exp2(S*c - m*c) with c = s_eff*log2(e).
//
// Softmax bookkeeping per query row: the exact running max (the "max"
// output) and a reference max used in the exponent.  The reference is only
// raised, and O and the sum rescaled, when a tile's max exceeds it by more
// than ln(256); so p <= 256 and the rescale is rare.  Each of the two lanes
// of a row keeps the max of its 16 keys; they are combined only when one
// passes the threshold, and for the output after the loop.  The sum is
// taken over the fp32 p, before they are rounded for the P.V contraction.
//
// Masks: kv_lengths and block lists cut whole tiles (tiles past the length,
// blocks not listed); element masks are applied only on tiles that need
// them (the ragged last tile, causal partial blocks); full blocks skip the
// mask.  A dense mask, a function of the key alone, is added to the logits
// by one more MFMA k-step (0 or -inf per key).  Masked logits are -inf
// internally; a row left with no valid key gets the page's uniform-weight
// result (mean of V over all K keys, max -1e9, lse -1e9 + ln K).
//
// Grid: one workgroup per (b, n, h, query tile), remapped so that each of the
// 8 XCDs walks a contiguous range of (b, h, n, q-tile) order: the q-tiles of
// one (n, h) share K/V in that XCD's L2 and a head's fp32 bias (shared by
// every n) stays resident there.  Within one (b, n, h) the q-tiles alternate
// between the two ends, which balances causal block masks across CUs.
#pragma once

// Internal: included by one translation unit per head dimension
// (kernel_mfma_d*.hip), each of which instantiates launch_d for its D.

#include <math.h>

#include "mfma_common.h"

namespace triattn {
namespace {

using namespace tile;


// Bias paths: none; staged through LDS by DMA; per-lane 4-byte loads (rows
// not 16-byte aligned).
enum BiasMode { kNoBias = 0, kBiasLds = 1, kBiasScalar = 2, kBiasLdsHalf = 3 };

// The bias in the inputs' 16-bit type (the page's newest kernels cast it so):
// a wave's 32 x 32 block is 32 rows of 64 bytes, DMA'd in two instructions
// of 16 rows.  Read back 8 bytes per lane (four keys) in the accumulator
// layout, 16-byte chunk g of row r stored at g ^ fbh(r): rows r, r+4, r+8,
// r+12 (the same banks) get distinct chunks, as do r and r+16.
constexpr int kBiasHalfRowBytes = kKTile * 2;
constexpr int kBiasHalfWaveBytes = 32 * kBiasHalfRowBytes;  // 2 KiB
constexpr int kBiasHalfDma = kBiasHalfWaveBytes / 1024;
__device__ __forceinline__ int fbh(int r) { return ((r >> 2) ^ (r >> 4)) & 3; }

// Kernel variant (a template value, not a mask kind of the calls) of block
// masks with 32- or 64-row query blocks, kept apart so that the per-tile
// tests of the block rows cost the whole-tile kernel nothing.
constexpr int kMaskBlockRows = 5;

// a block row's bitmaps with 32- or 64-row query blocks (kMultiWords)
__device__ __forceinline__ uint32_t* row_listed_bits(uint32_t* bits, int r) {
    return bits + kMultiWords * (1 + r);
}
__device__ __forceinline__ uint32_t* row_full_bits(uint32_t* bits, int r) {
    return bits + kMultiWords * (1 + kRowsMulti + r);
}

// Waves per SIMD the register budget must allow: four (128 VGPRs) for
// D <= 64, two for D = 128 (whose O accumulator alone takes 64 VGPRs).  At
// D = 64 a bias with a block-sparse mask, with a dense mask, or with a scale
// that is not a power of two needs more than 128 VGPRs (the block
// bookkeeping, the mask words, the bias / s products), and so does a dense
// mask with such a scale (the mask operands of the logits' MFMAs), and so
// does the variant for 32- / 64-row query blocks and 16-key blocks: those
// kernels run three waves instead of spilling.
template <int D, int KIND, int BIAS, bool EXACT>
constexpr int min_waves_per_simd() {
    if (D == 64 && BIAS != 0 &&
        (KIND == TRIATTN_MASK_BLOCK || KIND == kMaskBlockRows || KIND == TRIATTN_MASK_DENSE ||
         !EXACT))
        return 3;
    if (D == 64 && KIND == TRIATTN_MASK_DENSE && !EXACT) return 3;
    if (D == 64 && KIND == kMaskBlockRows) return 3;  // the per-wave block-row and 16-key state
    return D <= 64 ? 4 : D <= 128 ? 2 : 1;
}

template <typename T, int D, int KIND, int BIAS, bool EXACT, int W, bool PAD>
__global__ __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu(min_waves_per_simd<D, KIND, BIAS, EXACT>()))) void mfma_fwd_kernel(Params p) {
    using M = Mma<T>;
    using v8 = typename M::v8;
    using Ge = Geo<D>;
    constexpr int kWaves = W;
    constexpr int kThreads = 64 * W;
    constexpr int kQTile = 32 * W;  // query rows per workgroup
    // The K and V DMA instructions of a tile are dealt evenly to the waves,
    // so every wave has the same number in flight.
    constexpr int kDmaPerWave = 2 * Ge::kDma / W;
    static_assert(kDmaPerWave * W == 2 * Ge::kDma, "K/V DMAs split evenly over the waves");
    constexpr int kWords = static_cast<int>(kMaxKvBlocks / 32);
    constexpr bool kBlock = KIND == TRIATTN_MASK_BLOCK || KIND == kMaskBlockRows;
    constexpr bool kDense = KIND == TRIATTN_MASK_DENSE;
    constexpr bool kVarlen = KIND == kMaskVarlen;
    static_assert(!kVarlen || BIAS == kNoBias, "packed sequences carry no bias");
    // LDS: a ring of three buffers for K tiles and three for V tiles, and one
    // 32 x 32 fp32 bias block per wave (each wave refills its block as soon
    // as it has read it).  Every buffer is its own object, so the compiler
    // knows that a DMA into one buffer does not write the others and does
    // not wait for it before reading them.
    constexpr bool kBiasByDma = BIAS == kBiasLds || BIAS == kBiasLdsHalf;
    constexpr int kBiasBuf = BIAS == kBiasLds       ? kWaves * kBiasWaveBytes
                             : BIAS == kBiasLdsHalf ? kWaves * kBiasHalfWaveBytes
                                                    : 16;
    constexpr uint32_t kBiasElem = BIAS == kBiasLdsHalf ? 2u : 4u;  // bytes per bias element
    __shared__ __attribute__((aligned(1024))) char k_lds0[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds2[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds2[Ge::tileBytes];
    __shared__ __attribute__((aligned(1024))) char b_lds[kBiasBuf];
    // Block masks: bitmaps of the kv blocks listed and full for the
    // workgroup's block row.  Query blocks of 32 or 64 rows put 4 or 2
    // block rows in the 128 rows (each wave's 32 rows lie in one): the same
    // LDS then holds their union (the tiles visited) and a pair per block
    // row, of kMultiWords words each.
    __shared__ uint32_t block_bits[kBlock ? 2 * kWords : 1];
    uint32_t* const listed_bits = block_bits;
    uint32_t* const full_bits = block_bits + kWords;
    // after the key loop, the first K buffer holds the mean of V
    float* const mean_v = reinterpret_cast<float*>(k_lds0);
    static_assert(D * 4 <= Ge::tileBytes, "mean of V fits a K buffer");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
    const int col = lane & 31;  // this lane's query within the wave
    const int half = lane >> 5;

    // ---- workgroup -> (b, h, n, q tile), XCD-contiguous order ---------------
    const int64_t n_qt = (p.Q + kQTile - 1) / kQTile;
    const int64_t n_wg = gridDim.x;
    const int64_t w = blockIdx.x;
    const int64_t xcd = w % kXcds, slot = w / kXcds;
    const int64_t per = n_wg / kXcds, rem = n_wg % kXcds;
    const int64_t lid =
        xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    // Query tiles of one (b, n, h) are taken in the order 0, T-1, 1, T-2, ...
    // and every other (b, n, h) in the reverse of that.  Work per tile is the
    // same for dense masks and lengths, but with a causal block mask tile i
    // visits i + 1 blocks; when the whole grid is resident at once (512
    // workgroups at two per CU), this puts heavy and light tiles side by side
    // on a CU, whichever way the dispatcher fills its slots (consecutive
    // workgroups, or workgroups one round apart).
    const int64_t qr = lid % n_qt;
    const int64_t qt0 = (qr & 1) ? n_qt - 1 - qr / 2 : qr / 2;
    const int64_t qt = ((lid / n_qt) & 1) ? n_qt - 1 - qt0 : qt0;
    const int64_t n = (lid / n_qt) % p.N;
    const int64_t h = (lid / (n_qt * p.N)) % p.H;
    const int64_t b = lid / (n_qt * p.N * p.H);

    int K = static_cast<int>(p.K), Q = static_cast<int>(p.Q);
    const int64_t bnh = (b * p.N + n) * p.H + h;
    // Rows: (b, n, h) slices of Q x D and K x D elements, or, for packed
    // sequences, rows of q_rs / kv_rs elements from the sequence's first row.
    int64_t q_first = 0, k_first = 0;
    if constexpr (kVarlen) {
        const SeqRows sr = seq_rows(p, b);
        Q = static_cast<int>(sr.nq);
        K = static_cast<int>(sr.nk);
        q_first = sr.q0;
        k_first = sr.k0;
        if (qt * kQTile >= Q) return;  // the whole workgroup is past this sequence
    }
    // Dn: the head dimension of the data, D that of the tiles (with PAD, Dn <
    // D, a multiple of 8; without, Dn = D, so that every test of it below
    // folds away).  Columns Dn .. D-1 of Q, K and V enter the tiles as zeros:
    // they add nothing to Q.K, and the O columns they produce are not stored.
    const int Dn = PAD ? static_cast<int>(p.D) : D;
    const int64_t kv_rs = kVarlen ? p.kv_rs : Dn;  // K / V row stride (elements)
    const uint32_t kv_row_bytes = static_cast<uint32_t>(kv_rs * sizeof(T));
    const T* kbase = static_cast<const T*>(p.k) + (kVarlen ? k_first * kv_rs + h * Dn : bnh * p.K * Dn);
    const T* vbase = static_cast<const T*>(p.v) + (kVarlen ? k_first * kv_rs + h * Dn : bnh * p.K * Dn);
    const char* bslice =
        BIAS == kNoBias ? nullptr
                        : static_cast<const char*>(BIAS == kBiasLdsHalf ? p.bias16
                                                                        : static_cast<const void*>(p.bias)) +
                              (b * p.H + h) * p.Q * p.K * kBiasElem;
    const int q0 = static_cast<int>(qt) * kQTile;
    const int q0w = q0 + 32 * wave;
    const int qrow = q0w + col;  // this lane's query
    const bool row_ok = qrow < Q;
    const int qload = row_ok ? qrow : Q - 1;

    // Scale handling (see the header comment).
    const float zscale = EXACT ? 1.0f : p.scale;        // z = zscale * S
    const float c_exp = zscale * kLog2e;                 // exponent slope in S units
    const float lazy_s = kLazyLog / zscale;              // rescale threshold in S units
    const float inv_s = EXACT ? 1.0f : 1.0f / p.scale;   // bias -> S units

    // ---- visited key range / tile list -------------------------------
    int limit = K;  // keys >= limit are never valid
    // causal packed sequences: no row of this tile sees a key past its last row
    if (kVarlen && p.causal) limit = min(limit, q0 + kQTile);
    if (KIND == TRIATTN_MASK_KV_LENGTHS && p.kv_lengths) {
        const int64_t len = p.kv_lengths[b * p.N + n];
        limit = len < 0 ? 0 : (len > K ? K : static_cast<int>(len));
    }
    const int n_tiles = (limit + kKTile - 1) / kKTile;
    const int n_tiles_all = (K + kKTile - 1) / kKTile;
    int tiles_per_block = 1;
    constexpr bool multi_row = KIND == kMaskBlockRows;  // 32- or 64-row query blocks, 16-key blocks
    // 16-key kv blocks (only in that variant): tile t holds blocks 2t, 2t + 1
    const bool kv16 = multi_row && p.kv_block == 16;
    int wrow = 0;  // with multi_row: this wave's block row within the workgroup
    // (if constexpr keeps the block bitmaps out of the other kinds' LDS)
    if constexpr (kBlock) {
        tiles_per_block = kv16 ? 1 : static_cast<int>(p.kv_block / kKTile);
        const int words = static_cast<int>((p.n_kv_blocks + 31) / 32);
        const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
        if constexpr (!multi_row) {
            for (int i = tid; i < words; i += kThreads) {
                listed_bits[i] = 0u;
                full_bits[i] = 0u;
            }
            __syncthreads();
            const int64_t list_row = inst * p.n_q_rows + q0 / p.q_block;
            mark_list(listed_bits, p.kv_num_blocks, p.kv_indices, list_row, p.max_blocks,
                      p.n_kv_blocks, tid, kThreads);
            if (p.full_kv_num_blocks) {
                mark_list(full_bits, p.full_kv_num_blocks, p.full_kv_indices, list_row,
                          p.full_max_blocks, p.n_kv_blocks, tid, kThreads);
                mark_list(listed_bits, p.full_kv_num_blocks, p.full_kv_indices, list_row,
                          p.full_max_blocks, p.n_kv_blocks, tid, kThreads);
            }
        } else {
            const int qb = static_cast<int>(p.q_block);
            const bool split = qb < kQTileBlock;
            const int rows = split ? kQTileBlock / qb : 1;  // 2 or 4 block rows, or one
            wrow = split ? (32 * wave) / qb : 0;
            for (int i = tid; i < (1 + 2 * kRowsMulti) * kMultiWords; i += kThreads)
                block_bits[i] = 0u;
            __syncthreads();
            for (int r = 0; r < rows; ++r) {
                const int64_t qrow_blk = q0 / qb + r;
                if (qrow_blk >= p.n_q_rows) break;  // rows past Q
                const int64_t list_row = inst * p.n_q_rows + qrow_blk;
                mark_list(row_listed_bits(block_bits, r), p.kv_num_blocks, p.kv_indices, list_row,
                          p.max_blocks, p.n_kv_blocks, tid, kThreads);
                if (p.full_kv_num_blocks) {
                    mark_list(row_full_bits(block_bits, r), p.full_kv_num_blocks, p.full_kv_indices,
                              list_row, p.full_max_blocks, p.n_kv_blocks, tid, kThreads);
                    mark_list(row_listed_bits(block_bits, r), p.full_kv_num_blocks,
                              p.full_kv_indices, list_row, p.full_max_blocks, p.n_kv_blocks, tid,
                              kThreads);
                }
            }
            __syncthreads();
            for (int i = tid; i < words; i += kThreads) {
                uint32_t u = 0u;
                for (int r = 0; r < rows; ++r) u |= row_listed_bits(block_bits, r)[i];
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
            if (kv16) return blk < 0 ? -1 : static_cast<int>(blk >> 1);
            return blk < 0 ? -1 : static_cast<int>(blk) * tiles_per_block;
        }
    };
    auto next_tile = [&](int t) -> int {
        if (t < 0) return -1;
        if constexpr (!kBlock) {
            return t + 1 < n_tiles ? t + 1 : -1;
        } else {
            if (kv16) {  // tile t holds blocks 2t and 2t + 1
                const int64_t blk = next_set(listed_bits, 2 * static_cast<int64_t>(t) + 2, p.n_kv_blocks);
                return blk < 0 ? -1 : static_cast<int>(blk >> 1);
            }
            if ((t + 1) % tiles_per_block != 0 && t + 1 < n_tiles_all) return t + 1;
            const int64_t blk = next_set(listed_bits, t / tiles_per_block + 1, p.n_kv_blocks);
            return blk < 0 ? -1 : static_cast<int>(blk) * tiles_per_block;
        }
    };

    // ---- Q^T operand: registers for the whole key loop ----------------
    v8 qop[D / 16];
    {
        const T* qp = static_cast<const T*>(p.q) +
                      (kVarlen ? (q_first + qload) * p.q_rs + h * Dn : (bnh * p.Q + qload) * Dn) +
                      8 * half;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            // this lane's 8 columns 16 st + 8 half ..; zeros past Dn (the
            // load is unconditional, from the row's first columns there, so
            // that the four loads stay in flight together)
            const bool in_row = 16 * st + 8 * half < Dn;
            const u32x4 raw = *reinterpret_cast<const u32x4*>(qp + (in_row ? 16 * st : -8 * half));
            v8 x = __builtin_bit_cast(v8, in_row ? raw : u32x4{0u, 0u, 0u, 0u});
            if (EXACT) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = static_cast<T>(static_cast<float>(x[j]) * p.scale);
            }
            qop[st] = x;
        }
    }

    // ---- LDS regions and DMA address tables ------------------------------
    // rows past K read as zeros (the buffer range check)
    const uint32_t kv_bytes = kVarlen ? static_cast<uint32_t>(K) * kv_row_bytes
                                      : static_cast<uint32_t>(p.K * Dn * sizeof(T));
    const uint32_t kv_tile_bytes = kKTile * kv_row_bytes;  // one tile of K or V rows in memory
    const uint32_t bias_bytes = BIAS != kNoBias ? static_cast<uint32_t>(p.Q * p.K * kBiasElem) : 0u;
    // A DMA of tile t goes through a descriptor whose base is moved to the
    // tile and whose size shrinks by as much, so that the range check still
    // ends where the slice does, and a missing tile (t < 0) gets size 0 and
    // reads zeros.  The per-lane offsets are then the same for every tile
    // and the per-tile arithmetic is scalar.
    auto tile_desc = [](const void* base, uint32_t bytes, int t, uint32_t stride) {
        t = __builtin_amdgcn_readfirstlane(t);  // wave-uniform already
        const uint32_t off = t >= 0 ? static_cast<uint32_t>(t) * stride : 0u;
        return make_desc(static_cast<const char*>(base) + off, t >= 0 ? bytes - off : 0u);
    };
    const __amdgpu_buffer_rsrc_t bias_rsrc = make_rsrc(bslice, bias_bytes);
    auto kbuf = [&](int x) { return (lds_char*)(x == 0 ? k_lds0 : x == 1 ? k_lds1 : k_lds2); };
    auto vbuf = [&](int x) { return (lds_char*)(x == 0 ? v_lds0 : x == 1 ? v_lds1 : v_lds2); };
    lds_char* const bias_lds =  // this wave's block
        (lds_char*)b_lds + wave * (BIAS == kBiasLdsHalf ? kBiasHalfWaveBytes : kBiasWaveBytes);

    // K/V DMA of one tile: instruction I (I < kDma: K, else V) is issued by
    // wave I % kWaves; lane l of it fills LDS slot s = 64 (I % kDma) + l of
    // that tile, i.e. row s / chunks, stored chunk s % chunks, which holds
    // source chunk (s % chunks) ^ f(row).  Every wave issues its
    // instructions for every position, with kNoTile when there is no tile,
    // so the count of DMAs in flight per position is fixed.
    // A source chunk at or past Dn / 8 (columns the data does not have)
    // reads at kNoTile and lands as zeros: every slice is under 2^31 bytes.
    uint32_t kv_src[kDmaPerWave];
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
        const int I = wave + kWaves * j;
        const bool is_v = I >= Ge::kDma;
        const int s = 64 * (I % Ge::kDma) + lane;
        const int r = s / Ge::chunks, c = s % Ge::chunks;
        const int sc = c ^ (is_v ? Ge::fv(r) : Ge::fk(r));
        kv_src[j] = 8 * sc < Dn ? static_cast<uint32_t>(r * kv_row_bytes + 16 * sc) : kNoTile;
    }
    auto dma_k = [&](int t, int x) {
        const u32x4 desc = tile_desc(kbase, kv_bytes, t, kv_tile_bytes);
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) {
            const int I = wave + kWaves * j;  // wave-uniform
            if (I < Ge::kDma) dma16(desc, kbuf(x) + 1024 * I, kv_src[j]);
        }
    };
    auto dma_v = [&](int t, int x) {
        const u32x4 desc = tile_desc(vbase, kv_bytes, t, kv_tile_bytes);
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j) {
            const int I = wave + kWaves * j;
            if (I >= Ge::kDma) dma16(desc, vbuf(x) + 1024 * (I - Ge::kDma), kv_src[j]);
        }
    };
    // Bias DMA: the wave's block is kBiasDma instructions of 8 rows x 128
    // bytes; lane l of instruction j fills row r = 8j + l/8, stored chunk
    // l%8, holding source chunk (l%8) ^ fb(r) = (l%8) ^ (l/16) ^ 4(j%2).
    // Rows past Q read past the slice and land as zeros; keys past K read
    // the next row (masked).
    const uint32_t b_row = static_cast<uint32_t>(q0w + (lane >> 3)) * static_cast<uint32_t>(K) * 4u;
    const uint32_t b_src_even = b_row + 16u * static_cast<uint32_t>((lane & 7) ^ (lane >> 4));
    const uint32_t b_src_odd = b_row + 16u * static_cast<uint32_t>((lane & 7) ^ (lane >> 4) ^ 4);
    // 16-bit bias: lane l of instruction j fills row 16j + l/4, stored chunk
    // l%4, from source chunk (l%4) ^ fbh(row) = (l%4) ^ ((l/16 ^ j) % 4).
    const uint32_t bh_row = static_cast<uint32_t>(q0w + (lane >> 2)) * static_cast<uint32_t>(K) * 2u;
    auto dma_bias = [&](int t) {  // t >= 0
        if (BIAS == kBiasLdsHalf) {
            const u32x4 desc = tile_desc(bslice, bias_bytes, t, kBiasHalfRowBytes);
#pragma unroll
            for (int j = 0; j < kBiasHalfDma; ++j) {
                const uint32_t rows = static_cast<uint32_t>(16 * j) * static_cast<uint32_t>(K) * 2u;
                const uint32_t chunk = static_cast<uint32_t>((lane & 3) ^ (((lane >> 4) ^ j) & 3));
                dma16(desc, bias_lds + 1024 * j, bh_row + rows + 16u * chunk);
            }
            return;
        }
        if (BIAS != kBiasLds) return;
        const u32x4 desc = tile_desc(bslice, bias_bytes, t, kBiasRowBytes);
#pragma unroll
        for (int j = 0; j < kBiasDma; ++j) {
            const uint32_t rows = static_cast<uint32_t>(8 * j) * static_cast<uint32_t>(K) * 4u;
            dma16(desc, bias_lds + 1024 * j, ((j & 1) ? b_src_odd : b_src_even) + rows);
        }
    };
    // Bias read into the accumulator layout: register 4g+e is key
    // 8g + 4half + e, i.e. source chunk 2g + half of row col.
    auto read_bias = [&](f32x16& dst) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int chunk = (2 * g + half) ^ fb(col);
            const f32x4 bv = __builtin_bit_cast(
                f32x4,
                *reinterpret_cast<const lds_u32x4*>(bias_lds + col * kBiasRowBytes + 16 * chunk));
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * g + e] = bv[e];
        }
    };
    // 16-bit bias block into the accumulator layout: register 4g+e is key
    // 8g + 4half + e, i.e. bytes 8half..8half+7 of chunk g of row col.
    auto read_bias_half = [&](f32x16& dst) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int chunk = g ^ fbh(col);
            const u32x2 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
                bias_lds + col * kBiasHalfRowBytes + 16 * chunk + 8 * half);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if constexpr (sizeof(T) == 2 && __is_same(T, __bf16)) {
                    // a bf16 is the high half of the fp32 with the same value
                    dst[4 * g + 2 * e] = __uint_as_float(w[e] << 16);
                    dst[4 * g + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                } else {
                    const uint32_t u = w[e];
                    const auto lo = static_cast<unsigned short>(u & 0xffffu);
                    const auto hi = static_cast<unsigned short>(u >> 16);
                    dst[4 * g + 2 * e] = static_cast<float>(__builtin_bit_cast(_Float16, lo));
                    dst[4 * g + 2 * e + 1] = static_cast<float>(__builtin_bit_cast(_Float16, hi));
                }
            }
        }
    };
    // Bias for K % 4 != 0 (rows not 16-byte aligned): plain per-lane loads.
    const uint32_t bias_lane_scalar =
        static_cast<uint32_t>(qload) * static_cast<uint32_t>(K) * 4u + 16u * half;

    auto load_bias_scalar = [&](int t, f32x16& dst) {
        const uint32_t base = bias_lane_scalar + static_cast<uint32_t>(t) * kKTile * 4u;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * g + e] = bload32(bias_rsrc, base + 4u * (8 * g + e));
    };

    // Per-lane LDS offsets of the operand reads (within a tile).
    // K: row col, source chunk 2st + half, stored at chunk (2st + half) ^
    // fk(col) = 2st ^ (half ^ fk(col)); the row, the chunk and its high
    // bits occupy disjoint bits of the offset, so the offset of k-step st is
    // k_base ^ 32st.
    const int k_base = col * Ge::rowBytes + 16 * (half ^ Ge::fk(col));
    // V (transposing read): lane s names row 16t + 8u + 4half + (s%16)/4 and
    // column 32db + 16((s/16)%2) + 4(s%4), i.e. byte 8(s%2) of source chunk
    // 4db + 2((s/16)%2) + (s%4)/2; lane l then receives V[key][32db + l%32]
    // for the 4 keys of its slots 4u..4u+3.  The swizzle of row r depends on
    // r % 8 only, which t and u do not change: they add (16t + 8u) rows.
    // As for K, the column block db only flips bits of the stored chunk:
    // the offset for db is v_base ^ 64db.
    const int v_base = [&] {
        const int r = 4 * half + ((lane & 15) >> 2);
        const int chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        return r * Ge::rowBytes + 16 * (chunk ^ Ge::fv(r)) + 8 * (lane & 1);
    }();
    // Dense key mask as bits: lane i of dense_word holds bit j = key
    // 32(64c + i) + j valid, for the chunk c = dense_chunk of 64 tiles.  The
    // loop reads a tile's word with one readlane, so it issues no memory
    // operation for the mask; a chunk is rebuilt from the byte mask (32
    // coalesced byte loads and ballots per 64 tiles) when the key loop
    // reaches it.  The loads of a rebuild are waited for at once.
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
                // the 64 lanes cover tiles t0 + i0 + 2j and t0 + i0 + 2j + 1
                const int key = (t0 + i0 + 2 * j) * kKTile + lane;
                v[j] = key < K && dense_row[key] != 0;
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

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_true = -INFINITY;  // exact running max of this row, S units
    float m_ref = -INFINITY;   // reference max of the exponent, S units
    float m_thr = -INFINITY;   // m_ref + the lazy-rescale margin
    float m_exp = 0.f;         // m_ref * c_exp (0 while m_ref is -inf)
    float l_run = 0.f;         // this lane's half of the running sum

    // At D = 64 the QK MFMAs of one tile are interleaved with the
    // exponentials of the previous one (softmax_pv below); at D = 32 and 128
    // that measured slower than issuing them as one group.  The per-lane
    // bias loads keep the grouped order: interleaved, their registers spill;
    // so do the block-sparse kernels with a bias (interleaved, the 16-bit
    // bias one spilled past 128 VGPRs).
    constexpr bool kInterleave = D == 64 && BIAS != kBiasScalar && !(kBlock && BIAS != kNoBias);

    // A dense mask enters the logits through the matrix core, as one more
    // k-step: its A operand holds, in element 0 of lanes 0-31 (key col of
    // the tile), 0 for a valid key and -inf for a masked one (keys past K
    // included), its B operand 1 in element 0 of lanes 0-31 (every query),
    // and every other element is 0.  S^T then gains exactly 0 or -inf in
    // each key row, with no per-element select.
    v8 ones_op{};
    if constexpr (kDense) ones_op[0] = half == 0 ? static_cast<T>(1.0f) : static_cast<T>(0.0f);
    auto dense_op = [&](int t) {
        if ((t >> 6) != dense_chunk) load_dense_chunk(t >> 6);
        const uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dense_word), t & 63));
        v8 a{};
        a[0] = half == 0 && ((w >> col) & 1u) == 0u ? static_cast<T>(-INFINITY) : static_cast<T>(0.0f);
        return a;
    };
    v8 mop{};  // the dense-mask operand of the logits being formed

    // S^T = K . Q^T + bias for tile t from K buffer x and this wave's bias
    // block.  qk_load reads the bias into s and the K operands into kop;
    // the key loop issues the MFMAs later, between the exponentials of the
    // previous tile (qk does both at once, for the first tile).
    v8 kop[D / 16];
    auto qk_load = [&](f32x16& s, int t, int x) {
        s = f32x16{};
        if (BIAS == kBiasLds) read_bias(s);
        if (BIAS == kBiasLdsHalf) read_bias_half(s);
        if (BIAS == kBiasScalar) load_bias_scalar(t, s);
        if (BIAS != kNoBias && !EXACT) s *= inv_s;
        const lds_char* kt = kbuf(x);
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            kop[st] = __builtin_bit_cast(v8, *reinterpret_cast<const lds_u32x4*>(kt + (k_base ^ (32 * st))));
        if constexpr (kDense) mop = t >= 0 ? dense_op(t) : v8{};
    };
    auto qk = [&](f32x16& s, int t, int x) {
        qk_load(s, t, x);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) s = M::run(kop[st], qop[st], s);
        if constexpr (kDense) s = M::run(mop, ones_op, s);
    };

    // Softmax of tile t (logits in s) and O^T += V^T . P^T from V buffer x.
    // Between the row max and the exponentials it calls dma() (this
    // position's DMAs, issued once the bias reads have long returned).  With
    // kInterleave the MFMAs of the next tile's logits (operands already in
    // kop and s_nxt) are interleaved with the exponentials, one MFMA per few
    // vector instructions, so that the matrix core runs them while the wave
    // keeps issuing the softmax instead of stalling on their dependent chain.
    auto softmax_pv = [&](f32x16& s, int t, int x, f32x16& s_nxt, auto dma) {
        const int k0 = t * kKTile;
        // ---- element mask (only on tiles that need one) -------------------
        // Register r holds key k0 + 8(r/4) + r%4 in lanes 0-31 and that key
        // + 4 in lanes 32-63, so the length and dense-mask tests are uniform
        // per wave half: they become one 64-bit lane mask per register,
        // built with scalar instructions and applied by one select.
        bool need_mask = k0 + kKTile > limit;
        bool causal = false;
        if constexpr (kDense) need_mask = false;  // (masked in the logits' MFMAs)
        bool unlisted = false;  // a tile visited for another block row of the workgroup
        uint32_t half_w = ~0u;  // 16-key blocks: the keys of the tile's listed blocks
        uint32_t causal_w = ~0u;  // 16-key blocks: the keys under the causal mask_mod
        if constexpr (multi_row) {
            if (kv16) {
                const uint32_t* rl = row_listed_bits(block_bits, wrow);
                const uint32_t* rf = row_full_bits(block_bits, wrow);
                const int b0 = 2 * t;
                const bool l0 = bit_set(rl, b0), l1 = bit_set(rl, b0 + 1);
                half_w = (l0 ? 0x0000ffffu : 0u) | (l1 ? 0xffff0000u : 0u);
                if (half_w != ~0u) need_mask = true;
                if (p.mask_mod == TRIATTN_MOD_CAUSAL && k0 + kKTile - 1 > q0w) {
                    causal_w = (l0 && !bit_set(rf, b0) ? 0x0000ffffu : 0u) |
                               (l1 && !bit_set(rf, b0 + 1) ? 0xffff0000u : 0u);
                    if (causal_w != 0u) {
                        causal = true;
                        need_mask = true;
                    }
                }
            }
        }
        if constexpr (kBlock) {
            const int blk = t / tiles_per_block;
            if (multi_row && kv16) {
                // (the 16-key halves above)
            } else if (multi_row && !bit_set(row_listed_bits(block_bits, wrow), blk)) {
                unlisted = true;
                need_mask = true;
            } else if (p.mask_mod == TRIATTN_MOD_CAUSAL &&
                       !bit_set(multi_row ? row_full_bits(block_bits, wrow) : full_bits, blk) &&
                       k0 + kKTile - 1 > q0w) {
                causal = true;
                need_mask = true;
            }
        }
        if constexpr (kVarlen) {
            if (p.causal && k0 + kKTile - 1 > q0w) {
                causal = true;
                need_mask = true;
            }
        }
        if (need_mask) {
            // bit i of w: key k0 + i passes the length and dense tests
            const int room = limit - k0;
            uint32_t w = room >= kKTile ? ~0u : room <= 0 ? 0u : (1u << room) - 1u;
            if constexpr (multi_row) {
                if (unlisted) w = 0u;
                w &= half_w;
            }
            // 16-key blocks: the causal test only on the keys of partial blocks
            const bool causal_all = causal && causal_w == ~0u;
            const bool causal_some = causal && causal_w != ~0u;  // (16-key blocks only)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ka = 8 * (r / 4) + (r % 4);  // key offset in lanes 0-31
                // lanes 0-31 take bit ka, lanes 32-63 bit ka + 4, each spread
                // over its 32 lanes by sign-extending the one-bit field
                const uint32_t lo = static_cast<uint32_t>(static_cast<int32_t>(w << (31 - ka)) >> 31);
                const uint32_t hi = static_cast<uint32_t>(static_cast<int32_t>(w << (27 - ka)) >> 31);
                bool ok = __builtin_amdgcn_inverse_ballot_w64(lo | (static_cast<uint64_t>(hi) << 32));
                if (causal_all) ok = ok && qrow >= k0 + ka + 4 * half;
                if constexpr (multi_row) {
                    if (causal_some) {
                        // the field of key ka (lanes 0-31) or ka + 4 (lanes 32-63)
                        const uint32_t clo = static_cast<uint32_t>(static_cast<int32_t>(causal_w << (31 - ka)) >> 31);
                        const uint32_t chi = static_cast<uint32_t>(static_cast<int32_t>(causal_w << (27 - ka)) >> 31);
                        const bool c = __builtin_amdgcn_inverse_ballot_w64(clo | (static_cast<uint64_t>(chi) << 32));
                        ok = ok && (!c || qrow >= k0 + ka + 4 * half);
                    }
                }
                s[r] = ok ? s[r] : -INFINITY;
            }
        }

        // ---- row max; lazily raised reference ------------------------------
        // a tree of three-input maxima (8 instructions for 16 values)
        const float m0 = vmax(vmax(s[0], s[1]), s[2]);
        const float m1 = vmax(vmax(s[3], s[4]), s[5]);
        const float m2 = vmax(vmax(s[6], s[7]), s[8]);
        const float m3 = vmax(vmax(s[9], s[10]), s[11]);
        const float m4 = vmax(vmax(s[12], s[13]), s[14]);
        float mloc = vmax(vmax(vmax(m0, m1), m2), vmax(vmax(m3, m4), s[15]));
        // The two lanes of a row hold 16 keys each; their maxima are combined
        // only when one of them passes the threshold (the same in both), and
        // m_true after the loop.
        m_true = vmax(m_true, mloc);
        if (__ballot(mloc > m_thr)) {  // false while mloc == -inf
            mloc = max_halves(mloc);
            const bool raise = mloc > m_thr;
            // lanes that do not raise keep alpha = 1 exactly (their m_ref may
            // still be -inf); a raising lane with m_ref = -inf gets alpha = 0
            const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref - mloc) * c_exp) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
            if (raise) {
                m_ref = mloc;
                m_thr = mloc + lazy_s;
                m_exp = mloc * c_exp;
            }
        }
        const float mb = m_exp;
        dma();

        // ---- probabilities, their fp32 sum, P^T operands (rounded) ---------
        // The sum must use the unrounded p: rounding each p to bf16 moves
        // lse by up to ~2^-9, past its tolerance on short rows.
        v8 pop[2];
        float psum;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * tt + j], c_exp, -mb));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * tt + j + 1], c_exp, -mb));
                psum = tt + j == 0 ? p0 + p1 : psum + (p0 + p1);
                pop[tt][j] = static_cast<T>(p0);
                pop[tt][j + 1] = static_cast<T>(p1);
            }
        l_run += psum;
        // ---- S^T of the next tile, interleaved with the code above ----------
        if constexpr (kInterleave) {
#pragma unroll
            for (int st = 0; st < D / 16; ++st) s_nxt = M::run(kop[st], qop[st], s_nxt);
            if constexpr (kDense) s_nxt = M::run(mop, ones_op, s_nxt);
            // scheduling pattern: (1 MFMA, 7 VALU) per k-step
#pragma unroll
            for (int i = 0; i < D / 16 + (kDense ? 1 : 0); ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
            }
        }

        // ---- O^T += V^T . P^T ----------------------------------------------
        const lds_char* vt = vbuf(x);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(vt + (v_base ^ (64 * db)) + 16 * tt * Ge::rowBytes));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(vt + (v_base ^ (64 * db)) + (16 * tt + 8) * Ge::rowBytes));
                const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                const v8 a = __builtin_bit_cast(v8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
                oacc[db] = M::run(a, pop[tt], oacc[db]);
            }
    };

    // ---- key loop ---------------------------------------------------------
    // Position j of the tile sequence t_0, t_1, ... keeps K(t_j) and V(t_j)
    // in ring buffers j % 3.  At position j the logits of cur = t_j are in
    // registers; the loop computes the logits of nxt = t_{j+1} (K buffer
    // (j+1) % 3, bias block) and the softmax and P.V of t_j (V buffer j % 3),
    // so the QK contraction of one tile overlaps the softmax of the previous
    // one.  With kInterleave it reads the operands of the logits of t_{j+1},
    // takes the row max of t_j, issues the DMAs and then runs the
    // exponentials of t_j with the QK MFMAs of t_{j+1} between them; when
    // there is no t_{j+1} those reads and MFMAs still run, on stale buffers
    // that no DMA is writing, and their result is never used: that keeps the
    // exponentials and the MFMAs in one scheduling region.  Otherwise the
    // QK MFMAs go first and the DMAs follow them.  K/V DMAs run two positions ahead (K of t_{j+3}, V of
    // t_{j+2}); the bias block is refilled with t_{j+2} right after the
    // logits of t_{j+1} have read it.  Each position first waits for all of
    // this wave's DMAs but the K/V ones of the previous position.
    constexpr int kKvInFlight = kDmaPerWave;  // K/V DMAs a wave issues per position
    f32x16 sa, sb;
    int cur = first_tile();
    int nxt = next_tile(cur);
    int nxt2 = next_tile(nxt);
    if (cur >= 0) {
        // prologue: K(t0), bias(t0) | K(t1), V(t0) | logits of t0 | bias(t1) |
        // K(t2), V(t1)
        if constexpr (kDense) load_dense_chunk(cur >> 6);  // before any DMA is in flight
        dma_k(cur, 0);
        if (kBiasByDma) dma_bias(cur);
        dma_k(nxt, 1);
        dma_v(cur, 0);
        wait_vmem();
        __syncthreads();
        qk(sa, cur, 0);
        if (kBiasByDma && nxt >= 0) {
            wait_lds();  // the bias reads are done before the block is refilled
            dma_bias(nxt);
        }
        dma_k(nxt2, 2);
        dma_v(nxt, 1);
    }
    auto step = [&](auto X, f32x16& s_cur, f32x16& s_nxt) {
        constexpr int x = decltype(X)::value;  // j % 3
        const int nxt3 = __builtin_amdgcn_readfirstlane(next_tile(nxt2));
        // Everything but the last position's K/V DMAs has landed: K(nxt),
        // V(cur) and the bias block of nxt, for every wave once all have
        // passed the barrier, which also means every wave is done with the
        // buffers refilled below.
        __builtin_amdgcn_s_waitcnt(kVmcntWait<kKvInFlight>());
        __syncthreads();
        auto dma = [&]() {  // this position's DMAs
            if (kBiasByDma && nxt2 >= 0) {
                wait_lds();
                dma_bias(nxt2);
            }
            dma_k(nxt3, x);           // K(t_j) was last read one position ago
            dma_v(nxt2, (x + 2) % 3);  // V(t_{j-1}) likewise
        };
        if constexpr (kInterleave) {
            qk_load(s_nxt, nxt, (x + 1) % 3);
            softmax_pv(s_cur, cur, x, s_nxt, dma);
        } else {
            if (nxt >= 0) qk(s_nxt, nxt, (x + 1) % 3);
            dma();
            softmax_pv(s_cur, cur, x, s_nxt, [] {});
        }
        cur = nxt;
        nxt = nxt2;
        nxt2 = nxt3;
    };
    while (cur >= 0) {
        step(Par<0>{}, sa, sb);
        if (cur < 0) break;
        step(Par<1>{}, sb, sa);
        if (cur < 0) break;
        step(Par<2>{}, sa, sb);
        if (cur < 0) break;
        step(Par<0>{}, sb, sa);
        if (cur < 0) break;
        step(Par<1>{}, sa, sb);
        if (cur < 0) break;
        step(Par<2>{}, sb, sa);
    }

    // ---- epilogue ---------------------------------------------------------
    const float l_tot = sum_halves(l_run);
    m_true = max_halves(m_true);
    const bool dead = m_true == -INFINITY;
    // Does any row of the workgroup lack a valid key?  The flag lives in a K
    // buffer: after this wave's DMAs have landed and every wave has left the
    // loop, the ring is free.
    wait_vmem();
    __syncthreads();
    int* const any_dead = reinterpret_cast<int*>(k_lds1);
    if (tid == 0) *any_dead = 0;
    __syncthreads();
    if (__ballot(dead && row_ok) && lane == 0) *any_dead = 1;
    __syncthreads();
    if (*any_dead) {
        // Some row saw no valid key: its weights are uniform over all K keys.
        // Thread (key phase ph, 16-byte chunk c) sums rows ph, ph + P, ...;
        // lanes holding the same chunk are then summed by shuffles, and the
        // per-wave partial sums in LDS.
        constexpr int kChunks = D / 8;
        constexpr int kPhases = kThreads / kChunks;
        const int c = tid % kChunks, ph = tid / kChunks;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int kk = ph; kk < K && 8 * c < Dn; kk += kPhases) {
            const v8 x = __builtin_bit_cast(
                v8, *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(kk) * kv_rs + 8 * c));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += static_cast<float>(x[e]);
        }
#pragma unroll
        for (int off = kChunks; off < 64; off <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
        float* const part = reinterpret_cast<float*>(k_lds2);  // kWaves x D partial sums
        static_assert(kWaves * D * 4 <= Ge::tileBytes, "partial sums fit a K buffer");
        if (lane < kChunks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) part[wave * D + 8 * lane + e] = acc[e];
        }
        __syncthreads();
        for (int d = tid; d < D; d += kThreads) {
            float sum = 0.f;
            for (int w2 = 0; w2 < kWaves; ++w2) sum += part[w2 * D + d];
            // (a packed sequence with no key at all averages nothing: 0)
            mean_v[d] = K > 0 ? sum / static_cast<float>(K) : 0.f;
        }
        __syncthreads();
    }
    if (!row_ok) return;
    T* orow = static_cast<T*>(p.out) +
              (kVarlen ? ((q_first + qrow) * p.H + h) * Dn : (bnh * p.Q + qrow) * Dn);
    const float inv = dead ? 0.f : 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * half;
            if (d0 >= Dn) continue;  // a padding column (Dn is a multiple of 8)
            T o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o4[e] = static_cast<T>(dead ? mean_v[d0 + e] : oacc[db][4 * g + e] * inv);
            *reinterpret_cast<u32x2*>(orow + d0) = __builtin_bit_cast(u32x2, o4);
        }
    if (half == 0) {
        const int64_t ridx = kVarlen ? (q_first + qrow) * p.H + h : bnh * p.Q + qrow;
        if (p.lse)
            p.lse[ridx] = dead ? kMaskedLogit + (K > 0 ? logf(static_cast<float>(K)) : 0.f)
                               : m_ref * zscale + logf(l_tot);
        if (p.mx) p.mx[ridx] = dead ? kMaskedLogit : m_true * zscale;
    }
}

// Waves per workgroup.  The kernel also runs with 8 (256 query rows sharing
// each K/V tile, half the K/V bytes per wave); on the kv_lengths workload at
// D = 64 that measured no faster than 4, which wastes fewer rows when Q is
// not a multiple of 256, so 4 is used.
template <int D, int KIND>
constexpr int waves_of() {
    return 4;
}

template <typename T, int D, int KIND, int BIAS>
hipError_t launch_bias(const Params& p, bool exact, hipStream_t stream) {
    constexpr int W = waves_of<D, KIND>();
    const int64_t n_qt = (p.Q + 32 * W - 1) / (32 * W);
    const int64_t groups = p.B * p.N * p.H * n_qt;
    if (groups > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(groups));
    // head dimensions between the tile widths take the padded instantiation
    if (p.D != D) {
        if (exact)
            hipLaunchKernelGGL((mfma_fwd_kernel<T, D, KIND, BIAS, true, W, true>), grid, dim3(64 * W),
                               0, stream, p);
        else
            hipLaunchKernelGGL((mfma_fwd_kernel<T, D, KIND, BIAS, false, W, true>), grid, dim3(64 * W),
                               0, stream, p);
        return hipGetLastError();
    }
    if (exact)
        hipLaunchKernelGGL((mfma_fwd_kernel<T, D, KIND, BIAS, true, W, false>), grid, dim3(64 * W), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((mfma_fwd_kernel<T, D, KIND, BIAS, false, W, false>), grid, dim3(64 * W),
                           0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, int KIND>
hipError_t launch_kind(const Params& p, bool exact, hipStream_t stream) {
    if constexpr (KIND == kMaskVarlen) {
        return launch_bias<T, D, KIND, kNoBias>(p, exact, stream);  // no bias
    } else {
        // 16-bit bias (rows 16-byte aligned: checked by mfma_supports)
        if (p.bias16) return launch_bias<T, D, KIND, kBiasLdsHalf>(p, exact, stream);
        if (!p.bias) return launch_bias<T, D, KIND, kNoBias>(p, exact, stream);
        // The DMA path moves 16-byte chunks of bias rows: rows must be 16-byte
        // aligned.
        const bool rows16 = p.K % 4 == 0 && reinterpret_cast<uintptr_t>(p.bias) % 16 == 0;
        if (rows16) return launch_bias<T, D, KIND, kBiasLds>(p, exact, stream);
        return launch_bias<T, D, KIND, kBiasScalar>(p, exact, stream);
    }
}

template <typename T, int D>
hipError_t launch_d(const Params& p, bool exact, hipStream_t stream) {
    switch (p.mask_kind) {
    case TRIATTN_MASK_NONE:  // a kv_lengths mask with no lengths: limit = K
    case TRIATTN_MASK_KV_LENGTHS:
        return launch_kind<T, D, TRIATTN_MASK_KV_LENGTHS>(p, exact, stream);
    case TRIATTN_MASK_DENSE:
        return launch_kind<T, D, TRIATTN_MASK_DENSE>(p, exact, stream);
    case TRIATTN_MASK_BLOCK:
        if (p.q_block < kQTileBlock || p.kv_block < kKTile)
            return launch_kind<T, D, kMaskBlockRows>(p, exact, stream);
        return launch_kind<T, D, TRIATTN_MASK_BLOCK>(p, exact, stream);
    case kMaskVarlen:
        return launch_kind<T, D, kMaskVarlen>(p, exact, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace triattn
