// Dispatch of the MFMA forward kernel (mfma_fwd.h): which calls it serves,
// and the head dimension's instantiation to launch (kernel_mfma_d*.hip, one
// translation unit per D so that they compile in parallel).
#include <math.h>

#include "mfma_common.h"

namespace triattn {

using tile::kKTile;
using tile::kQTileBlock;
using tile::scale_is_exact;

bool mfma_supports(const Params& p, int32_t dtype) {
    if (dtype != TRIATTN_BF16 && dtype != TRIATTN_F16) return false;
    // Any multiple of 8 up to 256 runs on the tiles of the next width of 32,
    // 64, 128 or 256 (zero columns).
    if (p.D % 8 != 0 || p.D < 8 || p.D > 256) return false;
    // a 16-bit bias goes by DMA: its rows must be 16-byte aligned
    if (p.bias16 && (p.K % 8 != 0 || reinterpret_cast<uintptr_t>(p.bias16) % 16 != 0))
        return false;
    if (p.mask_kind == TRIATTN_MASK_BLOCK) {
        // whole 128-row tiles per block, or 2 or 4 blocks of 64 / 32 rows
        // per tile (each wave's 32 rows in one block); kv blocks of whole
        // 32-key tiles, or of 16 keys (two per tile).  Both exceptions take
        // bitmaps of kMultiWords x 32 kv blocks.
        const bool q_split = p.q_block % kQTileBlock != 0, kv16 = p.kv_block == 16;
        if (p.kv_block % kKTile != 0 && !kv16) return false;
        if (q_split && p.q_block != 64 && p.q_block != 32) return false;
        if ((q_split || kv16) && p.n_kv_blocks > tile::kMultiWords * 32) return false;
    }
    // Byte offsets within one (b, n, h) or (b, h) slice, including the
    // overhang of a ragged last tile and of the last query tile, must fit
    // the 32-bit per-lane offset.
    const int64_t kpad = (p.K + kKTile - 1) / kKTile * kKTile;
    const int64_t qpad = (p.Q + 255) / 256 * 256;  // the largest query tile
    const int64_t lim = int64_t(1) << 31;
    // packed sequences: K / V rows are kv_rs elements apart
    const int64_t kv_row = p.mask_kind == kMaskVarlen ? p.kv_rs : p.D;
    if (kpad * kv_row * 2 >= lim || qpad * p.D * 2 >= lim || (qpad + 1) * kpad * 4 >= lim)
        return false;
    // Other scales run as z = s * (Q.K + B/s): a negative s would flip the
    // max and a tiny one would overflow B/s; the generic kernel takes both.
    if (!scale_is_exact(p.scale) && !(p.scale >= 0x1p-40f)) return false;
    return true;
}

bool bwd_mfma_supports(const Params& p, int32_t dtype) {
    if (dtype != TRIATTN_BF16 && dtype != TRIATTN_F16) return false;
    // any multiple of 8 up to 128, on the tiles of the next width of 32, 64
    // or 128 (zero columns)
    if (p.D % 8 != 0 || p.D < 8 || p.D > 128) return false;
    if (p.mask_kind != TRIATTN_MASK_NONE && p.mask_kind != TRIATTN_MASK_KV_LENGTHS &&
        p.mask_kind != TRIATTN_MASK_DENSE && p.mask_kind != TRIATTN_MASK_BLOCK)
        return false;
    // the dK / dV kernel keeps one bit per 32-row query tile in a wave's
    // 64 lanes of 32 bits
    if (p.Q > 65536) return false;
    if (p.mask_kind == TRIATTN_MASK_BLOCK) {
        // dQ: one block row per 128-row workgroup, or 2 or 4 of 64 / 32 rows
        // (each wave's 32 rows in one; their bitmaps hold kMultiWords x 32
        // kv blocks); dK / dV: whole 32-row query tiles per block and one kv
        // block per wave
        if (p.kv_block % kKTile != 0) return false;
        if (p.q_block % 128 != 0 &&
            ((p.q_block != 64 && p.q_block != 32) || p.n_kv_blocks > tile::kMultiWords * 32))
            return false;
        if (p.n_q_rows > 2048 || p.n_kv_blocks > kMaxKvBlocks) return false;
    }
    const int64_t kpad = (p.K + 127) / 128 * 128;
    const int64_t qpad = (p.Q + 127) / 128 * 128;
    const int64_t lim = int64_t(1) << 31;
    if (kpad * p.D * 2 >= lim || qpad * p.D * 2 >= lim || (qpad + 32) * kpad * 4 >= lim ||
        qpad * 8 >= lim)
        return false;
    if (!scale_is_exact(p.scale) && !(p.scale >= 0x1p-40f)) return false;
    return true;
}

hipError_t launch_mfma(const Params& p, int32_t dtype, hipStream_t stream) {
    const bool exact = scale_is_exact(p.scale);
    if (p.D <= 32) return launch_mfma_d32(p, dtype, exact, stream);
    if (p.D <= 64) return launch_mfma_d64(p, dtype, exact, stream);
    if (p.D <= 128) return launch_mfma_d128(p, dtype, exact, stream);
    if (p.D <= 256) return launch_mfma_d256(p, dtype, exact, stream);
    return hipErrorInvalidValue;
}

}  // namespace triattn
