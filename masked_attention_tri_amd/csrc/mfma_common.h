// Building blocks shared by the MFMA forward kernels (gfx950): vector
// types, the MFMA wrappers, LDS tile geometry and swizzles, buffer
// descriptors, the inline-assembly LDS DMA and its waits, and the lane
// reductions of the S^T accumulator layout.  Internal to libtriattn.
#pragma once

#include <math.h>

#include "triattn_internal.h"

namespace triattn {
namespace tile {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kKTile = 32;           // keys per K/V tile
constexpr int kQTileBlock = 128;  // query rows per workgroup with block masks
// Block masks with 32- or 64-row query blocks: the kv-block bitmaps of the
// up to four block rows of a workgroup share the LDS of the one-row bitmaps
// (2 x kMaxKvBlocks bits): the union of the rows' listed blocks, then each
// row's listed and full blocks, kMultiWords words apiece.
constexpr int kRowsMulti = kQTileBlock / 32;
constexpr int kMultiWords = static_cast<int>(2 * (kMaxKvBlocks / 32) / (1 + 2 * kRowsMulti));
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog = 5.545177444479562f;  // ln(256): largest p before a rescale


template <typename T>
struct Mma;
template <>
struct Mma<__bf16> {
    using v8 = bf16x8;
    static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma<_Float16> {
    using v8 = f16x8;
    static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// LDS geometry and XOR swizzles of one head dimension.  Rows are stored
// unpadded; the 16-byte chunk c of row r lives at chunk position c ^ f(r).
template <int D>
struct Geo {
    static constexpr int rowBytes = 2 * D;              // one K or V row
    static constexpr int chunks = D / 8;                 // 16-byte chunks per row
    static constexpr int tileBytes = kKTile * rowBytes;  // one K (or V) tile
    static constexpr int stageBytes = 2 * tileBytes;     // K + V
    // A stage is 2*tileBytes/1024 DMA instructions (K first, then V), dealt
    // round-robin to the waves.
    static constexpr int kDma = tileBytes / 1024;
    static_assert(kDma * 1024 == tileBytes, "whole DMA instructions per tile");
    // K is read 16 bytes per lane down consecutive rows at one chunk.  At
    // D <= 128 it takes the backward kernels' tile swizzle (rows r, r+4,
    // r+8, r+12 to distinct chunk groups, a function of r % 16): measured
    // with the LDS bank-conflict counter, it leaves no conflict at D = 32 and
    // 64, where the swizzles (r/2 ^ r/8) % 4 and (r + r/8) % 8 left 0.7 and
    // 0.9 conflict cycles per LDS instruction.  At D = 256 a row is two
    // 256-byte bank cycles and r % 16 spreads 16 rows over the chunks.
    static __device__ __forceinline__ int fk(int r) {
        static_assert(D == 32 || D == 64 || D == 128 || D == 256, "swizzles defined");
        if (D == 32) return (r >> 2) & 3;
        if (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
        if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
        return r & 15;
    }
    // V is read by ds_read_b64_tr_b16: each 16 lanes take 4 consecutive rows
    // (first one a multiple of 4) x 2 adjacent chunks, and 32 lanes 4 rows x
    // 4 adjacent chunks.
    static __device__ __forceinline__ int fv(int r) {
        if (D == 32) return r & 2;
        if (D == 64) return 2 * (r & 3) + ((r >> 2) & 1);
        return (r & 3) == 0 ? 0 : (r & 3) == 1 ? 6 : (r & 3) == 2 ? 12 : 10;
    }
};

// The per-wave bias block: 32 query rows x 32 keys of fp32 = 128-byte rows,
// read 16 bytes per lane down consecutive rows.  Of 16 lanes served
// together, the 8 even rows land on one half of the 64 banks and the 8 odd
// rows on the other, so the swizzle must differ across each of the two
// groups: (r >> 1) & 7 does.
constexpr int kBiasRowBytes = kKTile * 4;
constexpr int kBiasWaveBytes = 32 * kBiasRowBytes;  // 4 KiB
constexpr int kBiasDma = kBiasWaveBytes / 1024;
__device__ __forceinline__ int fb(int r) { return (r >> 1) & 7; }

// Buffer resources: a 128-bit scalar descriptor (base, size in bytes).  Word
// 3 selects 32-bit data format, untyped access.  The scalar offset of every
// access below is 0; the whole offset is per lane and range-checked.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kRsrcWord3);
}
__device__ __forceinline__ float bload32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
// The same descriptor as four dwords, for the DMA below.
__device__ __forceinline__ u32x4 make_desc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xFFFFu, bytes,
                 static_cast<uint32_t>(kRsrcWord3)};
}
// 16 bytes per lane from byte offset voff into LDS at dst + 16 * lane
// (buffer_load_dwordx4 ... lds; M0 holds the LDS address).  Written as
// inline assembly so that the compiler does not track these LDS writes: it
// would otherwise wait for every DMA in flight before any later LDS read,
// which defeats prefetching more than one tile ahead.  The key loop waits
// for them explicitly (vmcnt) and fences with barriers instead.
__device__ __forceinline__ void dma16(const u32x4& r, lds_char* dst, uint32_t voff) {
    // (dst is wave-uniform by construction; readfirstlane tells the compiler)
    const uint32_t lds = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(reinterpret_cast<uintptr_t>(dst))));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(r)
                 : "memory");
}
// Wait until this wave's vector-memory operations (the DMAs) have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// s_waitcnt immediate that waits until at most N vector-memory operations of
// this wave are outstanding (vmcnt: bits 3:0 and 15:14; lgkmcnt and expcnt
// left at their maxima).
template <int N>
constexpr int kVmcntWait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    return (N & 15) | ((N >> 4) << 14) | 0x0F70;
}

// IEEE maximum (NaN-propagating); lowers to v_maximum3_f32 chains without the
// NaN-quieting instructions fmaxf needs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Value of x in the partner lane (lane ^ 32) combined with x: both halves of
// the wave hold the same query column, each for half of the keys.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int V>
struct Par {
    static constexpr int value = V;
};

// An offset past every buffer's range: a DMA with it reads nothing (the
// buffer range check returns zeros) and only fills a dead LDS buffer.
constexpr uint32_t kNoTile = 0x80000000u;

// Block bitmaps in LDS: one bit per kv (or query) block.
__device__ __forceinline__ bool bit_set(const uint32_t* bits, int64_t i) {
    return (bits[i >> 5] >> (i & 31)) & 1u;
}

// First set bit at or after `from`, or -1.
__device__ inline int64_t next_set(const uint32_t* bits, int64_t from, int64_t n) {
    int64_t j = from;
    while (j < n) {
        const uint32_t w = bits[j >> 5] >> (j & 31);
        if (w) {
            const int64_t r = j + __builtin_ctz(w);
            return r < n ? r : -1;
        }
        j = (j | 31) + 1;
    }
    return -1;
}

__device__ inline void mark_list(uint32_t* bits, const int32_t* counts, const int32_t* ids,
                          int64_t list_row, int64_t width, int64_t n_blocks, int tid,
                          int n_threads) {
    int64_t count = counts[list_row];
    count = count < 0 ? 0 : (count > width ? width : count);
    const int32_t* row = ids + list_row * width;
    for (int64_t j = tid; j < count; j += n_threads) {
        const int64_t id = row[j];
        if (id >= 0 && id < n_blocks) atomicOr(&bits[id >> 5], 1u << (id & 31));
    }
}

// s*x is exact for every normal x of the input format when s is 0 or a power
// of two with |s| <= 1 (so s*x cannot overflow).  An fp16 product that falls
// below the normal range is rounded to a subnormal, an absolute error of at
// most 2^-25 per element of Q, far below the output tolerance.
inline bool scale_is_exact(float s) {
    if (s == 0.0f) return true;
    int e = 0;
    return std::fabs(std::frexp(s, &e)) == 0.5f && std::fabs(s) <= 1.0f;
}

}  // namespace tile
}  // namespace triattn
