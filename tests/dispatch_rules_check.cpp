// Host driver for the C ABI's host rules (csrc/dispatch_rules.h) and the fused
// launch geometry (csrc/fused_geometry.h), built with AddressSanitizer and
// UndefinedBehaviorSanitizer (unsigned overflow included) by
// tests/test_dispatch_rules.py. Nothing here touches a GPU: the pointers are
// made-up addresses that are only compared, never dereferenced.
//
// 1. Fixed cases: sizes whose byte count wraps size_t, buffers that would run
//    past the end of the address space, and the layout of 8 ranks of such
//    sizes are rejected with AR_ERR_SHAPE by every entry point's rules.
// 2. Random adversarial params (extreme sizes, dtypes, rank counts, hidden
//    sizes, eps, pointers near 0 and near the top of the address space): every
//    accepted call satisfies the invariants the kernels rely on (the byte
//    count fits, every buffer lies inside the address space, outputs overlap
//    no input except exactly, slices stay inside [0, N) and partition it).
// 3. The fused geometry for every row width and extreme row counts.
// Prints "ok <checks>" and exits 0, or the first failed check and exits 1.
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "dispatch_rules.h"
#include "fused_geometry.h"

namespace {

unsigned long long g_checks = 0;

#define CHECK(cond, ...)                                        \
    do {                                                        \
        ++g_checks;                                             \
        if (!(cond)) {                                          \
            printf("FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
            printf(__VA_ARGS__);                                \
            printf("\n");                                       \
            return false;                                       \
        }                                                       \
    } while (0)

// xorshift64 (shifts and xors only, so the overflow checker has nothing to flag)
unsigned long long g_state = 0x9E3779B97F4A7C15ull;
unsigned long long next_u64()
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return g_state;
}
template <class T, size_t K>
T pick(const T (&a)[K])
{
    return a[next_u64() % K];
}

const void *ptr(uintptr_t a) { return reinterpret_cast<const void *>(a); }
void *mptr(uintptr_t a) { return reinterpret_cast<void *>(a); }

constexpr uintptr_t kBase = 0x7F0000000000ull;  // 256-byte aligned, made up
constexpr size_t kMaxSize = SIZE_MAX;

ar_params_t sum_params(size_t n, int32_t dtype, int32_t ranks)
{
    ar_params_t p;
    memset(&p, 0, sizeof p);
    p.elts_total = n;
    p.ranks = ranks;
    p.dtype = dtype;
    for (int r = 0; r < AR_MAX_RANKS; ++r)
        p.input_buffer_ptrs[r] = ptr(kBase + (uintptr_t)r * (1ull << 36));
    p.local_output_buffer_ptr = mptr(kBase + 9 * (1ull << 36));
    return p;
}

ar_params_t fused_params(size_t n, int32_t dtype, int32_t ranks, int32_t hidden)
{
    ar_params_t p = sum_params(n, dtype, ranks);
    p.fusion_params.hidden_size = hidden;
    p.fusion_params.weight_buffer = ptr(kBase + 10 * (1ull << 36));
    p.fusion_params.bias_buffer = ptr(kBase + 11 * (1ull << 36));
    p.fusion_params.residual_buffer = ptr(kBase + 12 * (1ull << 36));
    p.fusion_params.intermediate_buffer = mptr(kBase + 13 * (1ull << 36));
    p.fusion_params.eps = 1e-5f;
    return p;
}

// Every rule an entry point applies before it would launch, for one params.
bool all_shape_errors(const ar_params_t &p, bool sum_too, bool fused_too)
{
    size_t b = 7, e = 7;
    if (sum_too) {
        CHECK(ar_host::validate_sum(&p) == AR_ERR_SHAPE, "n=%zu", p.elts_total);
        CHECK(ar_host::configuration_supported(&p, AR_FUSION_NONE) == AR_ERR_SHAPE, "n=%zu", p.elts_total);
        CHECK(ar_host::slice_range_checked(&p, AR_FUSION_NONE, 0, 2, &b, &e) == AR_ERR_SHAPE, "n=%zu",
              p.elts_total);
        CHECK(b == 7 && e == 7, "outputs touched on error");
    }
    if (fused_too) {
        CHECK(ar_host::validate_fused(&p) == AR_ERR_SHAPE, "n=%zu", p.elts_total);
        CHECK(ar_host::configuration_supported(&p, AR_FUSION_RESIDUAL_RMS_NORM) == AR_ERR_SHAPE, "n=%zu",
              p.elts_total);
        CHECK(ar_host::slice_range_checked(&p, AR_FUSION_RESIDUAL_RMS_NORM, 1, 3, &b, &e) == AR_ERR_SHAPE, "n=%zu",
              p.elts_total);
        if (p.ranks == 1)
            CHECK(ar_host::validate_rmsnorm(&p) == AR_ERR_SHAPE, "n=%zu", p.elts_total);
    }
    return true;
}

bool fixed_cases()
{
    // byte counts that wrap size_t
    const size_t two62 = 1ull << 62;
    {
        ar_params_t p = sum_params(two62 + 16, AR_FP32, 2);
        if (!all_shape_errors(p, true, false))
            return false;
        p = fused_params(two62 + 16, AR_FP32, 2, 16);
        if (!all_shape_errors(p, true, true))
            return false;
        p = fused_params(two62, AR_FP32, 1, 1 << 20);
        if (!all_shape_errors(p, true, true))
            return false;
        p = sum_params(kMaxSize / 2 + 1, AR_FP16, 4);
        if (!all_shape_errors(p, true, false))
            return false;
        p = sum_params(kMaxSize / 2 + 1, AR_BF16, 8);
        if (!all_shape_errors(p, true, false))
            return false;
        p = sum_params(kMaxSize, AR_BF16, 3);
        if (!all_shape_errors(p, true, false))
            return false;
        p = sum_params(kMaxSize / 4 + 1, AR_FP32, 1);
        if (!all_shape_errors(p, true, false))
            return false;
    }
    // byte count fits, but a buffer would run past the end of the address space
    {
        ar_params_t p = sum_params(1ull << 40, AR_FP16, 2);
        p.local_output_buffer_ptr = mptr((UINTPTR_MAX & ~uintptr_t(255)) - (1ull << 38));  // 2^41 bytes would wrap
        if (!all_shape_errors(p, true, false))
            return false;
        p = sum_params(1ull << 40, AR_FP16, 2);
        p.input_buffer_ptrs[1] = ptr((UINTPTR_MAX & ~uintptr_t(255)) - 256);
        if (!all_shape_errors(p, true, false))
            return false;
        p = fused_params(1ull << 40, AR_BF16, 4, 8192);
        p.fusion_params.residual_buffer = ptr(UINTPTR_MAX & ~uintptr_t(255));
        if (!all_shape_errors(p, false, true))
            return false;
        p = fused_params(1ull << 20, AR_BF16, 4, 1 << 20);
        p.fusion_params.weight_buffer = ptr(UINTPTR_MAX & ~uintptr_t(255));
        if (!all_shape_errors(p, false, true))
            return false;
    }
    // the same sizes just inside the bounds are accepted
    {
        ar_params_t p = sum_params(kMaxSize / 2 / 16, AR_FP16, 2);
        p.input_buffer_ptrs[0] = p.input_buffer_ptrs[1] = ptr(kBase);  // in place; inputs may coincide
        p.local_output_buffer_ptr = mptr(kBase);
        CHECK(ar_host::validate_sum(&p) == AR_OK, "large but representable");
        p = sum_params(1ull << 40, AR_FP16, 2);
        p.local_output_buffer_ptr = mptr(UINTPTR_MAX - (1ull << 41) - 255);  // ends 256 bytes below the top
        CHECK(ar_host::validate_sum(&p) == AR_OK, "buffer ending at the top of the address space");
    }
    // layout: 8 ranks of a size whose slots do not fit size_t
    {
        size_t offs[AR_MAX_RANKS] = {0}, total = 7;
        CHECK(ar_host::partials_layout(two62 + 1, AR_FP32, 8, offs, &total) == AR_ERR_SHAPE, "fp32 2^62+1");
        CHECK(total == 7, "total touched on error");
        CHECK(ar_host::partials_layout(two62 / 8, AR_FP32, 8, offs, &total) == AR_ERR_SHAPE, "ranks * stride wraps");
        CHECK(ar_host::partials_layout(kMaxSize / 2, AR_FP16, 1, offs, &total) == AR_ERR_SHAPE, "round-up wraps");
        CHECK(ar_host::partials_layout(kMaxSize / 2 + 1, AR_FP16, 1, offs, &total) == AR_ERR_SHAPE, "bytes wrap");
        CHECK(ar_host::partials_layout(two62 / 16, AR_FP32, 8, offs, &total) == AR_OK, "fits");
        CHECK(total == 8 * (offs[1] - offs[0]), "total");
    }
    // slices of the largest representable sum: no wrap, exact partition
    {
        ar_params_t p = sum_params(kMaxSize / 2 - 128, AR_FP16, 2);
        p.input_buffer_ptrs[0] = ptr(256);
        p.input_buffer_ptrs[1] = ptr(256);
        p.local_output_buffer_ptr = mptr(256);  // in place
        CHECK(ar_host::validate_sum(&p) == AR_OK, "in-place sum of SIZE_MAX/2 - 128 fp16 elements");
        for (int S : {1, 2, 3, 7, 1023, 1024}) {
            size_t prev = 0;
            for (int k = 0; k < S; ++k) {
                size_t b = 0, e = 0;
                CHECK(ar_host::slice_range_checked(&p, AR_FUSION_NONE, k, S, &b, &e) == AR_OK, "S=%d k=%d", S, k);
                CHECK(b == prev && b <= e && e <= p.elts_total, "S=%d k=%d b=%zu e=%zu", S, k, b, e);
                CHECK(b == p.elts_total || b % 8 == 0, "aligned start");
                prev = e;
            }
            CHECK(prev == p.elts_total, "S=%d covers [0, N)", S);
        }
    }
    // NULL params and NULL outputs
    {
        size_t b = 0, e = 0, offs[1], total = 0;
        CHECK(ar_host::validate_sum(nullptr) == AR_ERR_NULL, "null");
        CHECK(ar_host::validate_fused(nullptr) == AR_ERR_NULL, "null");
        CHECK(ar_host::validate_rmsnorm(nullptr) == AR_ERR_NULL, "null");
        CHECK(ar_host::configuration_supported(nullptr, 0) == AR_ERR_NULL, "null");
        CHECK(ar_host::slice_range_checked(nullptr, 0, 0, 1, &b, &e) == AR_ERR_NULL, "null");
        ar_params_t p = sum_params(100, AR_FP16, 2);
        CHECK(ar_host::slice_range_checked(&p, 0, 0, 1, nullptr, &e) == AR_ERR_NULL, "null begin");
        CHECK(ar_host::partials_layout(1, AR_FP16, 1, nullptr, &total) == AR_ERR_NULL, "null offsets");
        CHECK(ar_host::partials_layout(1, AR_FP16, 1, offs, nullptr) == AR_ERR_NULL, "null total");
    }
    return true;
}

bool range_ok(const void *q, size_t n)
{
    return !q || reinterpret_cast<uintptr_t>(q) <= UINTPTR_MAX - n;
}

// Exact interval overlap in 128-bit arithmetic, independent of the header's.
bool overlaps128(const void *p, size_t n, const void *q, size_t m)
{
    if (!p || !q || !n || !m)
        return false;
    const unsigned __int128 a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

// Invariants of an accepted call with work to do.
bool accepted_invariants(const ar_params_t &p, bool fused)
{
    const size_t s = p.dtype == AR_FP32 ? 4 : 2;
    const unsigned __int128 bytes128 = (unsigned __int128)p.elts_total * s;
    CHECK(bytes128 <= SIZE_MAX, "accepted n=%zu s=%zu wraps", p.elts_total, s);
    const size_t bytes = p.elts_total * s;
    CHECK(p.ranks >= 1 && p.ranks <= AR_MAX_RANKS, "ranks %d", p.ranks);
    CHECK(p.local_output_buffer_ptr && range_ok(p.local_output_buffer_ptr, bytes), "output range");
    for (int r = 0; r < p.ranks; ++r) {
        CHECK(p.input_buffer_ptrs[r] && range_ok(p.input_buffer_ptrs[r], bytes), "input %d range", r);
        CHECK(reinterpret_cast<uintptr_t>(p.input_buffer_ptrs[r]) % s == 0, "input %d alignment", r);
        CHECK(p.input_buffer_ptrs[r] == p.local_output_buffer_ptr ||
                  !overlaps128(p.input_buffer_ptrs[r], bytes, p.local_output_buffer_ptr, bytes),
              "output partly overlaps input %d", r);
    }
    if (fused) {
        const ar_fusion_params_t &f = p.fusion_params;
        CHECK(f.hidden_size > 0 && p.elts_total % (size_t)f.hidden_size == 0, "shape");
        CHECK(f.eps >= 0.0f && !isinf(f.eps), "eps");
        const size_t hb = (size_t)f.hidden_size * s;
        CHECK(f.intermediate_buffer && range_ok(f.intermediate_buffer, bytes), "intermediate range");
        CHECK(f.weight_buffer && range_ok(f.weight_buffer, hb), "weight range");
        CHECK(range_ok(f.bias_buffer, hb) && range_ok(f.residual_buffer, bytes), "bias/residual range");
        CHECK(!overlaps128(p.local_output_buffer_ptr, bytes, f.intermediate_buffer, bytes), "out/inter overlap");
        for (const void *o : {(const void *)p.local_output_buffer_ptr, (const void *)f.intermediate_buffer}) {
            CHECK(!overlaps128(o, bytes, f.weight_buffer, hb) && !overlaps128(o, bytes, f.bias_buffer, hb),
                  "output overlaps weight or bias");
            CHECK(o == f.residual_buffer || !overlaps128(o, bytes, f.residual_buffer, bytes), "residual overlap");
        }
    }
    // slices partition [0, N) (whole rows for the fused op)
    const int32_t op = fused ? AR_FUSION_RESIDUAL_RMS_NORM : AR_FUSION_NONE;
    const int S = 1 + (int)(next_u64() % 9);
    size_t prev = 0;
    for (int k = 0; k < S; ++k) {
        size_t b = 0, e = 0;
        CHECK(ar_host::slice_range_checked(&p, op, k, S, &b, &e) == AR_OK, "slice");
        CHECK(b == prev && b <= e && e <= p.elts_total, "slice %d of %d: [%zu, %zu)", k, S, b, e);
        if (fused)
            CHECK(b % (size_t)p.fusion_params.hidden_size == 0, "whole rows");
        else
            CHECK(b == p.elts_total || (b * s) % 16 == 0, "16-byte slice start");
        if (b < e) {
            const ar_params_t q = ar_host::sliced(&p, op, b, e);
            CHECK(q.elts_total == e - b, "sliced size");
            CHECK(fused ? ar_host::validate_fused(&q) == AR_OK : ar_host::validate_sum(&q) == AR_OK,
                  "a slice of a valid call is valid");
        }
        prev = e;
    }
    CHECK(prev == p.elts_total, "slices cover [0, N)");
    return true;
}

bool random_cases(int iters)
{
    const size_t sizes[] = {0, 1, 2, 7, 8, 15, 16, 1000003, 1ull << 31, (1ull << 31) + 1003, 1ull << 40,
                            (1ull << 62) - 8, 1ull << 62, (1ull << 62) + 16, kMaxSize / 4, kMaxSize / 4 + 1,
                            kMaxSize / 2, kMaxSize / 2 + 1, kMaxSize - 15, kMaxSize};
    const int32_t dtypes[] = {AR_FP32, AR_FP16, AR_BF16, -1, 3, INT32_MIN, INT32_MAX};
    const int32_t ranks[] = {INT32_MIN, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, INT32_MAX};
    const int32_t hiddens[] = {INT32_MIN, -1, 0, 1, 7, 8, 256, 4096, 5120, 8192, 1 << 20, INT32_MAX};
    const float epss[] = {0.0f, -0.0f, 1e-6f, 1e-5f, FLT_MAX, FLT_MIN, -FLT_MIN, -1.0f, INFINITY, -INFINITY, NAN};
    const uintptr_t bases[] = {0, 1, 2, 16, 256, kBase, kBase + 2, kBase + 8, kBase + 16, kBase + (1ull << 20),
                               kBase + (1ull << 44), UINTPTR_MAX & ~uintptr_t(255),
                               (UINTPTR_MAX & ~uintptr_t(255)) - (1ull << 32), UINTPTR_MAX - 1,
                               (uintptr_t)1 << 63};
    unsigned long long accepted = 0;
    for (int it = 0; it < iters; ++it) {
        ar_params_t p;
        memset(&p, 0, sizeof p);
        p.elts_total = pick(sizes);
        if (next_u64() % 4 == 0)
            p.elts_total = next_u64() >> (next_u64() % 64);
        p.dtype = pick(dtypes);
        p.ranks = pick(ranks);
        // pointers: distinct 2^45-spaced regions, or shared/adversarial ones
        auto pointer = [&](int slot) -> uintptr_t {
            switch (next_u64() % 10) {
            case 0: return pick(bases);
            case 1: return 0;
            case 2:
            case 3:
            case 4: return kBase + (uintptr_t)slot * (1ull << 45);
            default: return kBase + (uintptr_t)slot * (1ull << 45) + (next_u64() % 64) * 2;
            }
        };
        for (int r = 0; r < AR_MAX_RANKS; ++r)
            p.input_buffer_ptrs[r] = ptr(pointer(r));
        p.local_output_buffer_ptr = mptr(next_u64() % 5 == 0 ? (uintptr_t)p.input_buffer_ptrs[0] : pointer(8));
        ar_fusion_params_t &f = p.fusion_params;
        f.hidden_size = pick(hiddens);
        if (next_u64() % 3 == 0 && p.elts_total > 0 && p.elts_total <= (size_t)INT32_MAX)
            f.hidden_size = (int32_t)p.elts_total;
        f.eps = pick(epss);
        f.weight_buffer = ptr(pointer(9));
        f.bias_buffer = next_u64() % 2 ? ptr(pointer(10)) : nullptr;
        f.residual_buffer = next_u64() % 2 ? ptr(pointer(11)) : nullptr;
        f.intermediate_buffer = mptr(next_u64() % 6 == 0 && f.residual_buffer ? (uintptr_t)f.residual_buffer
                                                                              : pointer(12));

        const int32_t st_sum = ar_host::validate_sum(&p), st_fused = ar_host::validate_fused(&p);
        const int32_t cs_sum = ar_host::configuration_supported(&p, AR_FUSION_NONE);
        const int32_t cs_fused = ar_host::configuration_supported(&p, AR_FUSION_RESIDUAL_RMS_NORM);
        CHECK(st_sum != AR_OK ? cs_sum == st_sum : (cs_sum == 0 || cs_sum == 1), "configuration_supported(NONE) %d vs %d",
              cs_sum, st_sum);
        CHECK(st_fused != AR_OK ? cs_fused == st_fused : (cs_fused == 0 || cs_fused == 1), "fused cs");
        CHECK(ar_host::validate_rmsnorm(&p) == (p.ranks != 1 ? AR_ERR_RANKS : st_fused), "rmsnorm rules");
        CHECK(ar_host::configuration_supported(&p, 2) == AR_ERR_SHAPE, "unknown op");
        if (st_sum == AR_OK && p.elts_total > 0) {
            ++accepted;
            if (!accepted_invariants(p, false))
                return false;
        }
        if (st_fused == AR_OK && p.elts_total > 0) {
            ++accepted;
            if (!accepted_invariants(p, true))
                return false;
        }
        // slice arguments out of range never pass
        size_t b = 0, e = 0;
        const int32_t bad_slice[][2] = {{0, 0}, {-1, 2}, {2, 2}, {0, 1025}, {INT32_MIN, 3}, {0, INT32_MAX}};
        const int32_t *bs = bad_slice[next_u64() % 6];
        const int32_t sr = ar_host::slice_range_checked(&p, AR_FUSION_NONE, bs[0], bs[1], &b, &e);
        CHECK(sr == (st_sum != AR_OK ? st_sum : AR_ERR_SLICE), "bad slice args: %d", sr);
        // layout of the same size
        size_t offs[AR_MAX_RANKS], total = 0;
        const int32_t lr = ar_host::partials_layout(p.elts_total, p.dtype, p.ranks, offs, &total);
        if (lr == AR_OK) {
            const size_t s = p.dtype == AR_FP32 ? 4 : 2;
            CHECK((unsigned __int128)p.elts_total * s * (unsigned)p.ranks <= total, "layout holds the partials");
            for (int r = 0; r < p.ranks; ++r) {
                CHECK(offs[r] % AR_SLOT_ALIGN_BYTES == 0, "slot alignment");
                CHECK(offs[r] <= total - p.elts_total * s, "slot inside the allocation");
                if (r > 0)
                    CHECK(offs[r] - offs[r - 1] >= p.elts_total * s + AR_SLOT_STAGGER_BYTES, "slots apart");
            }
        } else {
            CHECK(lr == AR_ERR_DTYPE || lr == AR_ERR_RANKS || lr == AR_ERR_SHAPE, "layout status %d", lr);
        }
    }
    CHECK(accepted > (unsigned long long)iters / 100, "too few accepted cases (%llu) to mean anything", accepted);
    return true;
}

bool geometry_cases()
{
    const size_t rows[] = {0, 1, 2, 191, 192, 193, 255, 256, 257, 1u << 20, (size_t)1 << 40, SIZE_MAX};
    const int cus[] = {1, 80, 256, 304, INT32_MAX};
    for (int ppr = 1; ppr <= 1 << 16; ppr += (ppr < 8192 ? 1 : 61)) {
        for (size_t r : rows)
            for (int c : cus) {
                const bool lat = ar_geometry::latency_layout(ppr, r, c);
                CHECK(!lat || r <= (size_t)c, "latency layout past the CU count");
                for (bool wide : {false, true}) {
                    const ar_geometry::FusedGeometry g = ar_geometry::fused_geometry(ppr, lat, wide);
                    CHECK(g.threads >= 64 && g.threads % 64 == 0 && g.threads <= g.bound, "ppr=%d", ppr);
                    CHECK(g.ppt == 0 || (size_t)g.ppt * g.threads * g.rows >= (size_t)ppr, "covers ppr=%d", ppr);
                    if (g.ppt > 0)
                        (void)ar_geometry::pipeline_mode(g.ppt, g.threads, ppr);
                }
            }
    }
    return true;
}

}  // namespace

int main()
{
    if (!fixed_cases() || !random_cases(400000) || !geometry_cases())
        return 1;
    printf("ok %llu\n", g_checks);
    return 0;
}
