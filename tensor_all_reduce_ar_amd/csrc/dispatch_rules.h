// dispatch_rules.h - the host-side rules of the C ABI (host code only): argument
// validation, the choice between the 16-byte vector path and the element-wise
// path, the two-shot slice arithmetic and the partials layout. Nothing here
// makes a HIP call or touches device memory; ar.hip's entry points call these
// functions before any launch, and a host test drives them with extreme and
// adversarial arguments under AddressSanitizer and UndefinedBehaviorSanitizer
// (unsigned overflow included).
//
// The checks follow "allreduce.d2" (configurationSupported, before the
// dispatch chain) and the fields of "type.d2" AllReduceParams /
// AllReduceFusionParams. Size rules: every full-size buffer holds elts_total
// elements, so elts_total * sizeof(T) must be representable in size_t, and
// every buffer's byte range [ptr, ptr + bytes) must lie inside the address
// space; a call that breaks either is AR_ERR_SHAPE (no such buffer can exist).
#ifndef AR_DISPATCH_RULES_H
#define AR_DISPATCH_RULES_H

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "ar.h"

namespace ar_host {

constexpr size_t kPackBytes = 16;
constexpr int32_t kMaxSlices = 1024;

inline bool valid_dtype(int32_t dtype) { return dtype == AR_FP32 || dtype == AR_FP16 || dtype == AR_BF16; }

inline size_t elem_size(int32_t dtype) { return dtype == AR_FP32 ? 4 : 2; }

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// n elements of `size` bytes: the byte count, or false if it does not fit size_t.
inline bool byte_count(size_t n, size_t size, size_t *bytes)
{
    if (n > SIZE_MAX / size)
        return false;
    *bytes = n * size;
    return true;
}

// [p, p + n) does not run past the end of the address space (NULL: nothing to check).
inline bool in_address_space(const void *p, size_t n)
{
    return !p || reinterpret_cast<uintptr_t>(p) <= UINTPTR_MAX - n;
}

// Byte ranges [p, p+n) and [q, q+m) share a byte. Both ranges must satisfy
// in_address_space (so neither end wraps).
inline bool overlap(const void *p, size_t n, const void *q, size_t m)
{
    if (!p || !q || !n || !m)
        return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

// An output may coincide exactly with a full-size input, not overlap it partly.
inline bool bad_alias(const void *out, const void *in, size_t bytes)
{
    return in != out && overlap(out, bytes, in, bytes);
}

inline int32_t validate_common(const ar_params_t *p)
{
    if (!p)
        return AR_ERR_NULL;
    if (!valid_dtype(p->dtype))
        return AR_ERR_DTYPE;
    if (p->ranks < 1 || p->ranks > AR_MAX_RANKS)
        return AR_ERR_RANKS;
    return AR_OK;
}

// Fusion op NONE. elts_total == 0 is valid (a no-op) whatever the pointers.
inline int32_t validate_sum(const ar_params_t *p)
{
    int32_t st = validate_common(p);
    if (st != AR_OK || p->elts_total == 0)
        return st;
    const size_t s = elem_size(p->dtype);
    size_t bytes = 0;
    if (!byte_count(p->elts_total, s, &bytes))
        return AR_ERR_SHAPE;
    if (!p->local_output_buffer_ptr)
        return AR_ERR_NULL;
    for (int r = 0; r < p->ranks; ++r)
        if (!p->input_buffer_ptrs[r])
            return AR_ERR_NULL;
    if (!aligned(p->local_output_buffer_ptr, s))
        return AR_ERR_ALIGN;
    for (int r = 0; r < p->ranks; ++r)
        if (!aligned(p->input_buffer_ptrs[r], s))
            return AR_ERR_ALIGN;
    if (!in_address_space(p->local_output_buffer_ptr, bytes))
        return AR_ERR_SHAPE;
    for (int r = 0; r < p->ranks; ++r)
        if (!in_address_space(p->input_buffer_ptrs[r], bytes))
            return AR_ERR_SHAPE;
    for (int r = 0; r < p->ranks; ++r)
        if (bad_alias(p->local_output_buffer_ptr, p->input_buffer_ptrs[r], bytes))
            return AR_ERR_ALIAS;
    return AR_OK;
}

// Fusion op RESIDUAL_RMS_NORM. The shape and eps are checked even when
// elts_total == 0; the buffers only when there is work.
inline int32_t validate_fused(const ar_params_t *p)
{
    int32_t st = validate_common(p);
    if (st != AR_OK)
        return st;
    const ar_fusion_params_t &f = p->fusion_params;
    if (f.hidden_size <= 0 || p->elts_total % static_cast<size_t>(f.hidden_size) != 0)
        return AR_ERR_SHAPE;
    if (!(f.eps >= 0.0f) || isinf(f.eps))
        return AR_ERR_EPS;
    if (p->elts_total == 0)
        return AR_OK;
    const size_t s = elem_size(p->dtype);
    size_t bytes = 0;
    if (!byte_count(p->elts_total, s, &bytes))
        return AR_ERR_SHAPE;
    const size_t hbytes = static_cast<size_t>(f.hidden_size) * s;  // <= bytes
    void *out = p->local_output_buffer_ptr, *inter = f.intermediate_buffer;
    if (!out || !inter || !f.weight_buffer)
        return AR_ERR_NULL;
    for (int r = 0; r < p->ranks; ++r)
        if (!p->input_buffer_ptrs[r])
            return AR_ERR_NULL;
    const void *ptrs[] = {out, inter, f.weight_buffer, f.bias_buffer, f.residual_buffer};
    for (const void *q : ptrs)
        if (q && !aligned(q, s))
            return AR_ERR_ALIGN;
    for (int r = 0; r < p->ranks; ++r)
        if (!aligned(p->input_buffer_ptrs[r], s))
            return AR_ERR_ALIGN;
    if (!in_address_space(out, bytes) || !in_address_space(inter, bytes) ||
        !in_address_space(f.residual_buffer, bytes) || !in_address_space(f.weight_buffer, hbytes) ||
        !in_address_space(f.bias_buffer, hbytes))
        return AR_ERR_SHAPE;
    for (int r = 0; r < p->ranks; ++r)
        if (!in_address_space(p->input_buffer_ptrs[r], bytes))
            return AR_ERR_SHAPE;
    if (overlap(out, bytes, inter, bytes))
        return AR_ERR_ALIAS;
    for (void *o : {out, inter}) {
        for (int r = 0; r < p->ranks; ++r)
            if (bad_alias(o, p->input_buffer_ptrs[r], bytes))
                return AR_ERR_ALIAS;
        if (overlap(o, bytes, f.weight_buffer, hbytes) || overlap(o, bytes, f.bias_buffer, hbytes))
            return AR_ERR_ALIAS;
    }
    if (bad_alias(inter, f.residual_buffer, bytes) || bad_alias(out, f.residual_buffer, bytes))
        return AR_ERR_ALIAS;
    return AR_OK;
}

// The unfused path's norm step: the fused op on exactly one input.
inline int32_t validate_rmsnorm(const ar_params_t *p)
{
    if (p && p->ranks != 1)
        return AR_ERR_RANKS;
    return validate_fused(p);
}

// Validated sum params: every pointer 16-byte aligned -> the vector path.
inline bool sum_vector_ok(const ar_params_t *p)
{
    if (!aligned(p->local_output_buffer_ptr, kPackBytes))
        return false;
    for (int r = 0; r < p->ranks; ++r)
        if (!aligned(p->input_buffer_ptrs[r], kPackBytes))
            return false;
    return true;
}

// Validated fused params: row bytes a multiple of 16 and every buffer
// 16-byte aligned -> the 16-byte pack kernels.
inline bool fused_vector_ok(const ar_params_t *p)
{
    const ar_fusion_params_t &f = p->fusion_params;
    const size_t s = elem_size(p->dtype);
    if ((static_cast<size_t>(f.hidden_size) * s) % kPackBytes != 0)
        return false;
    const void *ptrs[] = {p->local_output_buffer_ptr, f.intermediate_buffer, f.weight_buffer, f.bias_buffer,
                          f.residual_buffer};
    for (const void *q : ptrs)
        if (q && !aligned(q, kPackBytes))
            return false;
    for (int r = 0; r < p->ranks; ++r)
        if (!aligned(p->input_buffer_ptrs[r], kPackBytes))
            return false;
    return true;
}

// "allreduce.d2" configurationSupported: 1 = vector path, 0 = element-wise
// path, < 0 = invalid.
inline int32_t configuration_supported(const ar_params_t *p, int32_t fusion_op)
{
    if (fusion_op == AR_FUSION_NONE) {
        int32_t st = validate_sum(p);
        if (st != AR_OK)
            return st;
        return (p->elts_total == 0 || p->ranks == 1 || sum_vector_ok(p)) ? 1 : 0;
    }
    if (fusion_op == AR_FUSION_RESIDUAL_RMS_NORM) {
        int32_t st = validate_fused(p);
        if (st != AR_OK)
            return st;
        return (p->elts_total == 0 || fused_vector_ok(p)) ? 1 : 0;
    }
    return AR_ERR_SHAPE;
}

// [*b, *e) = share k of S equal shares of `total` items, each share
// ceil(total / S) rounded up to a multiple of `unit`, clipped to total.
// Validated params have total <= SIZE_MAX / 2 (their byte count fits size_t,
// elements are at least 2 bytes), and k < S <= kMaxSlices, unit <= 8, so
// k * per <= total + S * unit and per + unit cannot wrap.
inline void share(size_t total, size_t S, size_t k, size_t unit, size_t *b, size_t *e)
{
    size_t per = total / S + (total % S != 0);
    per = (per + unit - 1) / unit * unit;
    const size_t start = k * per;
    *b = start < total ? start : total;
    *e = total - *b > per ? *b + per : total;
}

// Elements [begin, end) of slice `slice` of `num_slices` (two-shot split) on
// validated params. Sum: equal shares of ceil(N / S) elements rounded up to
// whole 16-byte packs, so every slice of a 16-byte-aligned buffer starts
// 16-byte aligned. Fused: equal shares of ceil(rows / S) whole rows.
inline int32_t slice_range(const ar_params_t *p, int32_t fusion_op, int32_t slice, int32_t num_slices, size_t *begin,
                           size_t *end)
{
    if (num_slices < 1 || num_slices > kMaxSlices || slice < 0 || slice >= num_slices)
        return AR_ERR_SLICE;
    const size_t S = static_cast<size_t>(num_slices), k = static_cast<size_t>(slice);
    if (fusion_op == AR_FUSION_NONE) {
        share(p->elts_total, S, k, kPackBytes / elem_size(p->dtype), begin, end);
        return AR_OK;
    }
    if (fusion_op != AR_FUSION_RESIDUAL_RMS_NORM)
        return AR_ERR_SHAPE;
    const size_t H = static_cast<size_t>(p->fusion_params.hidden_size);
    size_t r0 = 0, r1 = 0;
    share(p->elts_total / H, S, k, 1, &r0, &r1);
    *begin = r0 * H;  // <= elts_total
    *end = r1 * H;
    return AR_OK;
}

// The checked form of slice_range: validates p for the op first.
inline int32_t slice_range_checked(const ar_params_t *p, int32_t fusion_op, int32_t slice, int32_t num_slices,
                                   size_t *begin, size_t *end)
{
    if (!begin || !end)
        return AR_ERR_NULL;
    int32_t st = fusion_op == AR_FUSION_RESIDUAL_RMS_NORM ? validate_fused(p)
                 : fusion_op == AR_FUSION_NONE            ? validate_sum(p)
                                                          : AR_ERR_SHAPE;
    if (st != AR_OK)
        return st;
    return slice_range(p, fusion_op, slice, num_slices, begin, end);
}

// Params restricted to elements [begin, end) of params validated for
// `fusion_op`: every full-size buffer the op reads or writes is offset; bias
// and weight ([hidden]) are not, and the sum leaves fusion_params alone (it
// neither validates nor reads them).
inline ar_params_t sliced(const ar_params_t *p, int32_t fusion_op, size_t begin, size_t end)
{
    ar_params_t q = *p;
    const size_t off = begin * elem_size(p->dtype);  // begin <= elts_total, whose byte count fits
    auto at = [off](const void *b) -> const void * {
        return b ? static_cast<const void *>(static_cast<const char *>(b) + off) : nullptr;
    };
    for (int r = 0; r < p->ranks; ++r)
        q.input_buffer_ptrs[r] = at(p->input_buffer_ptrs[r]);
    q.local_output_buffer_ptr = const_cast<void *>(at(p->local_output_buffer_ptr));
    if (fusion_op == AR_FUSION_RESIDUAL_RMS_NORM) {
        q.fusion_params.residual_buffer = at(p->fusion_params.residual_buffer);
        q.fusion_params.intermediate_buffer = const_cast<void *>(at(p->fusion_params.intermediate_buffer));
    }
    q.elts_total = end - begin;
    return q;
}

// ar_partials_layout: slot r at r * stride, stride = round_up(bytes,
// AR_SLOT_ALIGN_BYTES) + AR_SLOT_STAGGER_BYTES; AR_ERR_SHAPE if the total does
// not fit size_t.
inline int32_t partials_layout(size_t elts_total, int32_t dtype, int32_t ranks, size_t *slot_offsets,
                               size_t *total_bytes)
{
    if (!valid_dtype(dtype))
        return AR_ERR_DTYPE;
    if (ranks < 1 || ranks > AR_MAX_RANKS)
        return AR_ERR_RANKS;
    if (!slot_offsets || !total_bytes)
        return AR_ERR_NULL;
    const size_t a = AR_SLOT_ALIGN_BYTES, stagger = AR_SLOT_STAGGER_BYTES, R = static_cast<size_t>(ranks);
    size_t bytes = 0;
    if (!byte_count(elts_total, elem_size(dtype), &bytes) || bytes > SIZE_MAX - (a - 1) - stagger)
        return AR_ERR_SHAPE;
    const size_t stride = (bytes + a - 1) / a * a + stagger;
    if (stride > SIZE_MAX / R)
        return AR_ERR_SHAPE;
    for (size_t r = 0; r < R; ++r)
        slot_offsets[r] = r * stride;
    *total_bytes = R * stride;
    return AR_OK;
}

}  // namespace ar_host

#endif  // AR_DISPATCH_RULES_H
