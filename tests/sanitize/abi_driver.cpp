// Drives the host-side validation of libtriattn's C ABI under
// AddressSanitizer / UndefinedBehaviorSanitizer (the host code of the C
// entry points and of the kernel dispatch, compiled for the host only, the
// launchers replaced by stubs that abort): tri_attn_check, tri_attn_fwd and
// tri_attn_fwd_bias_dtype with rejected or empty arguments,
// tri_attn_varlen_check / _fwd, tri_attn_bwd with rejected arguments,
// tri_attn_bwd_workspace_size, tri_attn_mask_to_kv_lengths
// and tri_attn_status_str, over sizes that overflow int64 products, negative
// sizes, bad enums, misaligned and missing pointers.  No call reaches a
// kernel launch: every one is rejected or has no work.  Device pointers are
// fake aligned addresses, never dereferenced on the host.  Exit status 0 when
// every status matches the documented one (a sanitizer report aborts).
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <limits>

#include "triattn.h"

static int failures = 0;
static void expect(const char* what, int got, int want) {
    if (got != want) {
        printf("%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

static void* const A = reinterpret_cast<void*>(uintptr_t(1) << 20);  // 16-byte aligned
static float* const F = reinterpret_cast<float*>(uintptr_t(1) << 21);

static tri_attn_shape shp(int64_t B, int64_t N, int64_t H, int64_t Q, int64_t K, int64_t D) {
    tri_attn_shape s{B, N, H, Q, K, D};
    return s;
}

int main() {
    const int64_t big = int64_t(1) << 40, huge = std::numeric_limits<int64_t>::max();
    const tri_attn_shape ok = shp(1, 2, 2, 8, 8, 64);
    const float nan = NAN;
    // ---- tri_attn_check ----------------------------------------------------
    expect("check ok", tri_attn_check(&ok, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, F, F), TRIATTN_OK);
    expect("check null shape", tri_attn_check(nullptr, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, F, F),
           TRIATTN_ERR_INVALID_ARG);
    const int64_t sizes[] = {-1, 0, 1, 7, big, huge};
    for (int64_t x : sizes) {
        for (int which = 0; which < 6; ++which) {
            tri_attn_shape s = ok;
            int64_t* f[6] = {&s.B, &s.N, &s.H, &s.Q, &s.K, &s.D};
            *f[which] = x;
            tri_attn_check(&s, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, F, F);
            tri_attn_check(&s, TRIATTN_F32, A, A, A, F, nullptr, 0.5f, A, nullptr, nullptr);
            tri_attn_bwd_workspace_size(&s, 1);
            tri_attn_bwd_workspace_size(&s, 0);
        }
    }
    tri_attn_shape all_big = shp(big, big, big, big, big, 64);
    expect("check overflow", tri_attn_check(&all_big, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, F, F),
           TRIATTN_ERR_UNSUPPORTED);
    expect("workspace overflow", static_cast<int>(tri_attn_bwd_workspace_size(&all_big, 1)), 0);
    expect("check dtype", tri_attn_check(&ok, 77, A, A, A, F, nullptr, nan, A, F, F), TRIATTN_ERR_INVALID_ARG);
    expect("check scale inf", tri_attn_check(&ok, TRIATTN_BF16, A, A, A, F, nullptr, INFINITY, A, F, F),
           TRIATTN_ERR_INVALID_ARG);
    expect("check misaligned q",
           tri_attn_check(&ok, TRIATTN_BF16, static_cast<char*>(A) + 2, A, A, F, nullptr, nan, A, F, F),
           TRIATTN_ERR_INVALID_ARG);
    tri_attn_shape d300 = shp(1, 1, 1, 8, 8, 300);
    expect("check D past envelope", tri_attn_check(&d300, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, F, F),
           TRIATTN_ERR_UNSUPPORTED);
    // masks
    tri_attn_mask m{};
    m.kind = 99;
    expect("mask kind", tri_attn_check(&ok, TRIATTN_BF16, A, A, A, F, &m, nan, A, F, F), TRIATTN_ERR_INVALID_ARG);
    m = tri_attn_mask{};
    m.kind = TRIATTN_MASK_BLOCK;
    m.kv_num_blocks = static_cast<const int32_t*>(A);
    m.kv_indices = static_cast<const int32_t*>(A);
    const int64_t blocks[] = {-5, 0, 1, 3, 8, 128, big, huge};
    for (int64_t qb : blocks)
        for (int64_t kb : blocks)
            for (int64_t mb : blocks) {
                m.q_block = qb;
                m.kv_block = kb;
                m.max_blocks = mb;
                m.full_max_blocks = mb;
                m.stride_b = qb;
                m.stride_n = kb;
                m.stride_h = mb;
                tri_attn_check(&ok, TRIATTN_BF16, A, A, A, F, &m, nan, A, F, F);
                tri_attn_check(&all_big, TRIATTN_BF16, A, A, A, F, &m, nan, A, F, F);
            }
    m = tri_attn_mask{};
    m.kind = TRIATTN_MASK_KV_LENGTHS;
    expect("lengths without array", tri_attn_check(&ok, TRIATTN_BF16, A, A, A, F, &m, nan, A, F, F),
           TRIATTN_ERR_INVALID_ARG);
    // fwd entry points: rejected (nothing launched) or no work
    expect("fwd rejected", tri_attn_fwd(&ok, 77, A, A, A, F, nullptr, nan, A, F, F, nullptr),
           TRIATTN_ERR_INVALID_ARG);
    tri_attn_shape empty = shp(1, 0, 2, 8, 8, 64);
    expect("fwd empty", tri_attn_fwd(&empty, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, F, F, nullptr),
           TRIATTN_OK);
    expect("fwd bias dtype rejected",
           tri_attn_fwd_bias_dtype(&ok, TRIATTN_BF16, A, A, A, A, TRIATTN_F16, nullptr, nan, A, F, F, nullptr),
           TRIATTN_ERR_INVALID_ARG);
    // ---- varlen -------------------------------------------------------------
    tri_attn_varlen d{};
    d.layout = TRIATTN_QKV_SEPARATE;
    d.mask_type = TRIATTN_VARLEN_PADDING;
    d.batch = 2;
    d.heads = 2;
    d.head_dim = 64;
    d.total_q = 10;
    d.total_kv = 12;
    d.cu_seqlens_q = static_cast<const int32_t*>(A);
    d.cu_seqlens_kv = static_cast<const int32_t*>(A);
    d.max_seqlen_q = 8;
    d.max_seqlen_kv = 8;
    expect("varlen ok", tri_attn_varlen_check(&d, TRIATTN_BF16, A, A, A, nan, A, nullptr, nullptr), TRIATTN_OK);
    for (int64_t x : sizes) {
        tri_attn_varlen e = d;
        e.total_q = x;
        tri_attn_varlen_check(&e, TRIATTN_BF16, A, A, A, nan, A, nullptr, nullptr);
        e = d;
        e.heads = x;
        e.max_seqlen_kv = x;
        tri_attn_varlen_check(&e, TRIATTN_BF16, A, A, A, nan, A, nullptr, nullptr);
        e = d;
        e.batch = x;
        e.head_dim = x;
        tri_attn_varlen_check(&e, TRIATTN_F16, A, A, A, nan, A, nullptr, nullptr);
    }
    d.layout = 9;
    expect("varlen layout", tri_attn_varlen_fwd(&d, TRIATTN_BF16, A, A, A, nan, A, nullptr, nullptr, nullptr),
           TRIATTN_ERR_INVALID_ARG);
    expect("varlen null", tri_attn_varlen_check(nullptr, TRIATTN_BF16, A, A, A, nan, A, nullptr, nullptr),
           TRIATTN_ERR_INVALID_ARG);
    // ---- backward ------------------------------------------------------------
    expect("bwd no workspace",
           tri_attn_bwd(&ok, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, A, F, F, A, A, A, F, nullptr, 0, nullptr),
           TRIATTN_ERR_INVALID_ARG);
    expect("bwd small workspace",
           tri_attn_bwd(&ok, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, A, F, F, A, A, A, F, F, 12, nullptr),
           TRIATTN_ERR_INVALID_ARG);
    expect("bwd overflow",
           tri_attn_bwd(&all_big, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, A, F, F, A, A, A, F, F, 1 << 20, nullptr),
           TRIATTN_ERR_UNSUPPORTED);
    expect("bwd empty",
           tri_attn_bwd(&empty, TRIATTN_BF16, A, A, A, F, nullptr, nan, A, A, F, F, A, A, A, F, nullptr, 0, nullptr),
           TRIATTN_OK);
    // ---- helpers -------------------------------------------------------------
    int32_t* I = static_cast<int32_t*>(A);
    expect("mask_to_kv_lengths K 0", tri_attn_mask_to_kv_lengths(static_cast<uint8_t*>(A), 4, 0, I, I, nullptr),
           TRIATTN_ERR_INVALID_ARG);
    expect("mask_to_kv_lengths overflow",
           tri_attn_mask_to_kv_lengths(static_cast<uint8_t*>(A), big, big, I, I, nullptr),
           TRIATTN_ERR_UNSUPPORTED);
    for (triattn_status st : {TRIATTN_OK, TRIATTN_ERR_INVALID_ARG, TRIATTN_ERR_UNSUPPORTED, TRIATTN_ERR_HIP})
        if (!tri_attn_status_str(st)) ++failures;
    printf(failures ? "abi driver: %d FAILED\n" : "abi driver: ok\n", failures);
    return failures != 0;
}
