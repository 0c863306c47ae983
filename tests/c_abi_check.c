/*
 * c_abi_check.c - drives libar.so through include/ar.h from plain C (no
 * Python, no torch): device memory and a stream from the HIP runtime's C API,
 * the calls of the boundary, and the CPU oracle (oracle/ar_oracle.c, linked in
 * as test infrastructure) for the expected values.
 *
 * Cases: a bf16 sum over 3 ranks of 10007 elements (a ragged tail), bitwise;
 * an fp16 fused op over 4 ranks, 37 rows of 640 with bias and residual, S
 * bitwise and the output within 2 ulp; an fp32 fused op over 2 ranks with the
 * intermediate written over the residual, S bitwise and the output within
 * 1e-5 relative; rejected calls (partial overlap, unknown dtype) that must
 * return their codes and leave the output untouched; the two-shot slices of
 * both ops, run one by one into the full buffers, against the unsliced
 * oracle result; the unfused path (ar_sum, then ar_rmsnorm on the rounded
 * sum) against the oracle's fused op on that rounded sum; ar_sum captured into
 * a HIP graph and replayed twice, with new input values written between the
 * replays; and the host-only calls.
 * Inputs are seeded: SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) on the
 * element index, mapped to a normal value by the Box-Muller transform.
 *
 * Prints "c_abi_check: OK" and exits 0, or names the failing case and exits 1.
 * Built by tests/c_abi_build.py; run by tests/test_gpu_c_abi.py.
 */
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ar.h"

/* oracle/ar_oracle.c */
int oracle_ar_sum(int dtype, int ranks, const void *const *parts, size_t n, void *out);
int oracle_ar_residual_rmsnorm(int dtype, int ranks, const void *const *parts, size_t n, int hidden,
                               const void *bias, const void *residual, const void *weight, float eps,
                               void *out, void *intermediate);
uint16_t oracle_f16_from_f64(double x);
uint16_t oracle_bf16_from_f64(double x);

static int failures = 0;

#define CHECK_HIP(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "c_abi_check: %s failed: %s\n", #call, hipGetErrorString(e_)); \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

static void fail(const char *what)
{
    fprintf(stderr, "c_abi_check: FAIL %s\n", what);
    ++failures;
}

static uint64_t splitmix64(uint64_t x)
{
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

/* Normal value of stream `seed` at index i: Box-Muller on two 53-bit uniforms. */
static double normal_at(uint64_t seed, uint64_t i, double mean, double var)
{
    const uint64_t a = splitmix64(seed * 0x100000001B3ull + 2 * i), b = splitmix64(seed * 0x100000001B3ull + 2 * i + 1);
    const double u1 = ((a >> 11) + 1.0) / 9007199254740993.0, u2 = (b >> 11) / 9007199254740992.0;
    return mean + sqrt(var) * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static size_t esize(int dtype) { return dtype == AR_FP32 ? 4 : 2; }

/* n values of stream `seed`, rounded to dtype, into a new host array. */
static void *host_values(int dtype, size_t n, uint64_t seed, double mean, double var)
{
    void *p = malloc(n * esize(dtype) + 1);
    for (size_t i = 0; i < n; ++i) {
        const double x = normal_at(seed, i, mean, var);
        if (dtype == AR_FP32)
            ((float *)p)[i] = (float)x;
        else if (dtype == AR_FP16)
            ((uint16_t *)p)[i] = oracle_f16_from_f64(x);
        else
            ((uint16_t *)p)[i] = oracle_bf16_from_f64(x);
    }
    return p;
}

/* A device buffer of `bytes`, holding a copy of `h` unless `h` is NULL. */
static void *to_device(const void *h, size_t bytes)
{
    void *d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
    if (h && bytes)
        CHECK_HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

/* Order-preserving integer of a 16-bit encoding (+0 and -0 map together). */
static int64_t ordered16(uint16_t b) { return (b & 0x8000) ? 0x8000 - (int64_t)b : (int64_t)b; }

static void compare(const char *what, int dtype, const void *got, const void *want, size_t n, int bitwise)
{
    size_t bad = 0;
    for (size_t i = 0; i < n; ++i) {
        if (dtype == AR_FP32) {
            uint32_t g, w;
            memcpy(&g, (const char *)got + 4 * i, 4);
            memcpy(&w, (const char *)want + 4 * i, 4);
            if (bitwise ? g != w
                        : fabs((double)((const float *)got)[i] - ((const float *)want)[i]) >
                              1e-5 * fabs((double)((const float *)want)[i]) + 1e-30)
                ++bad;
        } else {
            const uint16_t g = ((const uint16_t *)got)[i], w = ((const uint16_t *)want)[i];
            const int64_t d = ordered16(g) - ordered16(w);
            if (bitwise ? g != w : (d > 2 || d < -2))
                ++bad;
        }
    }
    if (bad) {
        char msg[160];
        snprintf(msg, sizeof msg, "%s: %zu of %zu elements differ", what, bad, n);
        fail(msg);
    }
}

static ar_params_t params(size_t n, int ranks, int dtype, void *const *parts, void *out)
{
    ar_params_t p;
    memset(&p, 0, sizeof p);
    p.elts_total = n;
    p.ranks = ranks;
    p.dtype = dtype;
    for (int r = 0; r < ranks; ++r)
        p.input_buffer_ptrs[r] = parts[r];
    p.local_output_buffer_ptr = out;
    return p;
}

static void check_sum(hipStream_t s)
{
    const int dt = AR_BF16, R = 3;
    const size_t n = 10007, bytes = n * esize(dt);
    void *h[R], *d[R];
    for (int r = 0; r < R; ++r) {
        h[r] = host_values(dt, n, 3101 + r, 0.0, 1.0 / R);
        d[r] = to_device(h[r], bytes);
    }
    void *dout = to_device(NULL, bytes), *got = malloc(bytes), *want = malloc(bytes);
    ar_params_t p = params(n, R, dt, d, dout);
    if (ar_sum(&p, s) != AR_OK)
        fail("ar_sum status");
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(got, dout, bytes, hipMemcpyDeviceToHost));
    if (oracle_ar_sum(dt, R, (const void *const *)h, n, want) != 0)
        fail("oracle_ar_sum status");
    compare("bf16 sum, 3 ranks, 10007 elements", dt, got, want, n, 1);

    /* rejected: an output that starts 32 bytes into a partial (a partial
       overlap), and an unknown dtype; the output keeps its bits */
    memset(got, 0x5A, bytes);
    CHECK_HIP(hipMemcpy(dout, got, bytes, hipMemcpyHostToDevice));
    ar_params_t bad = params(n, R, dt, d, (char *)d[1] + 2 * 16);
    if (ar_sum(&bad, s) != AR_ERR_ALIAS)
        fail("partial overlap is not AR_ERR_ALIAS");
    bad = params(n, R, 7, d, dout);
    if (ar_sum(&bad, s) != AR_ERR_DTYPE)
        fail("unknown dtype is not AR_ERR_DTYPE");
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(want, dout, bytes, hipMemcpyDeviceToHost));
    if (memcmp(got, want, bytes) != 0)
        fail("a rejected call wrote the output");
    if (!ar_status_string(AR_ERR_ALIAS) || !ar_status_string(-12345))
        fail("ar_status_string returned NULL");

    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipFree(d[r]));
        free(h[r]);
    }
    CHECK_HIP(hipFree(dout));
    free(got);
    free(want);
}

/* Fused op; with `inter_is_residual` the intermediate is the residual buffer. */
static void check_fused(hipStream_t s, int dt, int R, size_t rows, int H, int with_bias, int inter_is_residual,
                        const char *what)
{
    const size_t n = rows * (size_t)H, bytes = n * esize(dt), hb = (size_t)H * esize(dt);
    const float eps = 1e-6f;
    void *h[AR_MAX_RANKS], *d[AR_MAX_RANKS];
    for (int r = 0; r < R; ++r) {
        h[r] = host_values(dt, n, 3201 + r, 0.0, 1.0 / R);
        d[r] = to_device(h[r], bytes);
    }
    void *hb_bias = with_bias ? host_values(dt, H, 3300, 0.0, 0.02) : NULL;
    void *hres = host_values(dt, n, 3301, 0.0, 1.0), *hw = host_values(dt, H, 3302, 1.0, 0.1);
    void *dbias = with_bias ? to_device(hb_bias, hb) : NULL, *dres = to_device(hres, bytes), *dw = to_device(hw, hb);
    void *dout = to_device(NULL, bytes), *dinter = inter_is_residual ? dres : to_device(NULL, bytes);

    ar_params_t p = params(n, R, dt, d, dout);
    p.fusion_params.bias_buffer = dbias;
    p.fusion_params.residual_buffer = dres;
    p.fusion_params.hidden_size = H;
    p.fusion_params.weight_buffer = dw;
    p.fusion_params.eps = eps;
    p.fusion_params.intermediate_buffer = dinter;
    if (ar_configuration_supported(&p, AR_FUSION_RESIDUAL_RMS_NORM) < 0)
        fail("ar_configuration_supported rejected a valid fused call");
    if (ar_workspace_size(&p) != 0)
        fail("ar_workspace_size is not 0");
    if (ar_residual_rmsnorm(&p, s) != AR_OK)
        fail("ar_residual_rmsnorm status");
    CHECK_HIP(hipStreamSynchronize(s));

    void *got_out = malloc(bytes), *got_inter = malloc(bytes), *want_out = malloc(bytes), *want_inter = malloc(bytes);
    CHECK_HIP(hipMemcpy(got_out, dout, bytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(got_inter, dinter, bytes, hipMemcpyDeviceToHost));
    if (oracle_ar_residual_rmsnorm(dt, R, (const void *const *)h, n, H, hb_bias, hres, hw, eps, want_out,
                                   want_inter) != 0)
        fail("oracle_ar_residual_rmsnorm status");
    char msg[160];
    snprintf(msg, sizeof msg, "%s: intermediate", what);
    compare(msg, dt, got_inter, want_inter, n, 1);
    snprintf(msg, sizeof msg, "%s: output", what);
    compare(msg, dt, got_out, want_out, n, 0);

    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipFree(d[r]));
        free(h[r]);
    }
    if (dbias)
        CHECK_HIP(hipFree(dbias));
    CHECK_HIP(hipFree(dres));
    CHECK_HIP(hipFree(dw));
    CHECK_HIP(hipFree(dout));
    if (!inter_is_residual)
        CHECK_HIP(hipFree(dinter));
    free(hb_bias);
    free(hres);
    free(hw);
    free(got_out);
    free(got_inter);
    free(want_out);
    free(want_inter);
}

/* Bytes of `n` elements of `dtype` read back from the device. */
static void *from_device(const void *d, size_t bytes)
{
    void *h = malloc(bytes ? bytes : 1);
    CHECK_HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    return h;
}

/* ar_sum_slice over 3 slices (bf16, 4 ranks, 10007 elements), each written
 * into the full output; ar_slice_range must tile [0, n) in order. */
static void check_sum_slices(hipStream_t s)
{
    const int dt = AR_BF16, R = 4, S = 3;
    const size_t n = 10007, bytes = n * esize(dt);
    void *h[R], *d[R];
    for (int r = 0; r < R; ++r) {
        h[r] = host_values(dt, n, 3401 + r, 0.0, 1.0 / R);
        d[r] = to_device(h[r], bytes);
    }
    void *fill = malloc(bytes), *want = malloc(bytes);
    memset(fill, 0x5A, bytes);
    void *dout = to_device(fill, bytes);
    ar_params_t p = params(n, R, dt, d, dout);
    size_t next = 0;
    for (int k = 0; k < S; ++k) {
        size_t b = 0, e = 0;
        if (ar_slice_range(&p, AR_FUSION_NONE, k, S, &b, &e) != AR_OK || b != next || e < b || e > n)
            fail("ar_slice_range does not tile the sum in order");
        next = e;
        if (ar_sum_slice(&p, k, S, s) != AR_OK)
            fail("ar_sum_slice status");
    }
    if (next != n)
        fail("ar_slice_range leaves the end of the sum uncovered");
    if (ar_sum_slice(&p, S, S, s) != AR_ERR_SLICE)
        fail("a slice index past the count is not AR_ERR_SLICE");
    CHECK_HIP(hipStreamSynchronize(s));
    void *got = from_device(dout, bytes);
    if (oracle_ar_sum(dt, R, (const void *const *)h, n, want) != 0)
        fail("oracle_ar_sum status");
    compare("bf16 sum from 3 slices, 4 ranks, 10007 elements", dt, got, want, n, 1);
    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipFree(d[r]));
        free(h[r]);
    }
    CHECK_HIP(hipFree(dout));
    free(fill);
    free(got);
    free(want);
}

/* Fused inputs of one case, on the host and on the device. */
typedef struct {
    int dt, R, H;
    size_t rows, n, bytes, hbytes;
    void *h[AR_MAX_RANKS], *d[AR_MAX_RANKS];
    void *hbias, *hres, *hw, *dbias, *dres, *dw;
} fused_case;

static void fused_case_make(fused_case *c, int dt, int R, size_t rows, int H, uint64_t seed)
{
    memset(c, 0, sizeof *c);
    c->dt = dt, c->R = R, c->H = H, c->rows = rows, c->n = rows * (size_t)H;
    c->bytes = c->n * esize(dt), c->hbytes = (size_t)H * esize(dt);
    for (int r = 0; r < R; ++r) {
        c->h[r] = host_values(dt, c->n, seed + r, 0.0, 1.0 / R);
        c->d[r] = to_device(c->h[r], c->bytes);
    }
    c->hbias = host_values(dt, H, seed + 100, 0.0, 0.02);
    c->hres = host_values(dt, c->n, seed + 101, 0.0, 1.0);
    c->hw = host_values(dt, H, seed + 102, 1.0, 0.1);
    c->dbias = to_device(c->hbias, c->hbytes);
    c->dres = to_device(c->hres, c->bytes);
    c->dw = to_device(c->hw, c->hbytes);
}

static void fused_case_free(fused_case *c)
{
    for (int r = 0; r < c->R; ++r) {
        CHECK_HIP(hipFree(c->d[r]));
        free(c->h[r]);
    }
    CHECK_HIP(hipFree(c->dbias));
    CHECK_HIP(hipFree(c->dres));
    CHECK_HIP(hipFree(c->dw));
    free(c->hbias);
    free(c->hres);
    free(c->hw);
}

static void set_fusion(ar_params_t *p, const fused_case *c, float eps, void *dinter)
{
    p->fusion_params.bias_buffer = c->dbias;
    p->fusion_params.residual_buffer = c->dres;
    p->fusion_params.hidden_size = c->H;
    p->fusion_params.weight_buffer = c->dw;
    p->fusion_params.eps = eps;
    p->fusion_params.intermediate_buffer = dinter;
}

/* ar_residual_rmsnorm_slice over 4 slices of whole rows (bf16, 3 ranks, 37
 * rows of 1536), each written into the full outputs. */
static void check_fused_slices(hipStream_t s)
{
    const int S = 4;
    const float eps = 1e-5f;
    fused_case c;
    fused_case_make(&c, AR_BF16, 3, 37, 1536, 3501);
    void *fill = malloc(c.bytes);
    memset(fill, 0x5A, c.bytes);
    void *dout = to_device(fill, c.bytes), *dinter = to_device(fill, c.bytes);
    ar_params_t p = params(c.n, c.R, c.dt, c.d, dout);
    set_fusion(&p, &c, eps, dinter);
    size_t next = 0;
    for (int k = 0; k < S; ++k) {
        size_t b = 0, e = 0;
        if (ar_slice_range(&p, AR_FUSION_RESIDUAL_RMS_NORM, k, S, &b, &e) != AR_OK || b != next || e < b ||
            b % (size_t)c.H || e % (size_t)c.H)
            fail("ar_slice_range does not tile the fused op in whole rows");
        next = e;
        if (ar_residual_rmsnorm_slice(&p, k, S, s) != AR_OK)
            fail("ar_residual_rmsnorm_slice status");
    }
    if (next != c.n)
        fail("ar_slice_range leaves rows of the fused op uncovered");
    CHECK_HIP(hipStreamSynchronize(s));
    void *got_out = from_device(dout, c.bytes), *got_inter = from_device(dinter, c.bytes);
    void *want_out = malloc(c.bytes), *want_inter = malloc(c.bytes);
    if (oracle_ar_residual_rmsnorm(c.dt, c.R, (const void *const *)c.h, c.n, c.H, c.hbias, c.hres, c.hw, eps, want_out,
                                   want_inter) != 0)
        fail("oracle_ar_residual_rmsnorm status");
    compare("bf16 fused from 4 slices, 3 ranks, 37 x 1536: intermediate", c.dt, got_inter, want_inter, c.n, 1);
    compare("bf16 fused from 4 slices, 3 ranks, 37 x 1536: output", c.dt, got_out, want_out, c.n, 0);
    CHECK_HIP(hipFree(dout));
    CHECK_HIP(hipFree(dinter));
    fused_case_free(&c);
    free(fill);
    free(got_out);
    free(got_inter);
    free(want_out);
    free(want_inter);
}

/* The unfused path: ar_sum to a buffer of T, then ar_rmsnorm on it. The
 * expected values are the oracle's fused op with one input, the oracle's
 * rounded sum. */
static void check_unfused(hipStream_t s)
{
    const float eps = 1e-6f;
    fused_case c;
    fused_case_make(&c, AR_FP16, 8, 16, 4096, 3601);
    void *dsum = to_device(NULL, c.bytes), *dout = to_device(NULL, c.bytes), *dinter = to_device(NULL, c.bytes);
    ar_params_t ps = params(c.n, c.R, c.dt, c.d, dsum);
    if (ar_sum(&ps, s) != AR_OK)
        fail("ar_sum status (unfused path)");
    void *x[1] = {dsum};
    ar_params_t pn = params(c.n, 1, c.dt, x, dout);
    set_fusion(&pn, &c, eps, dinter);
    if (ar_rmsnorm(&pn, s) != AR_OK)
        fail("ar_rmsnorm status");
    pn.ranks = 2;
    pn.input_buffer_ptrs[1] = dsum;
    if (ar_rmsnorm(&pn, s) != AR_ERR_RANKS)
        fail("ar_rmsnorm with 2 ranks is not AR_ERR_RANKS");
    CHECK_HIP(hipStreamSynchronize(s));
    void *got_out = from_device(dout, c.bytes), *got_inter = from_device(dinter, c.bytes);
    void *sum = malloc(c.bytes), *want_out = malloc(c.bytes), *want_inter = malloc(c.bytes);
    if (oracle_ar_sum(c.dt, c.R, (const void *const *)c.h, c.n, sum) != 0)
        fail("oracle_ar_sum status (unfused path)");
    const void *one[1] = {sum};
    if (oracle_ar_residual_rmsnorm(c.dt, 1, one, c.n, c.H, c.hbias, c.hres, c.hw, eps, want_out, want_inter) != 0)
        fail("oracle_ar_residual_rmsnorm status (unfused path)");
    compare("fp16 unfused path, 8 ranks, 16 x 4096: intermediate", c.dt, got_inter, want_inter, c.n, 1);
    compare("fp16 unfused path, 8 ranks, 16 x 4096: output", c.dt, got_out, want_out, c.n, 0);
    CHECK_HIP(hipFree(dsum));
    CHECK_HIP(hipFree(dout));
    CHECK_HIP(hipFree(dinter));
    fused_case_free(&c);
    free(got_out);
    free(got_inter);
    free(sum);
    free(want_out);
    free(want_inter);
}

/* ar_sum captured into a HIP graph on `s`, replayed twice; between the
 * replays the inputs get new values (same buffers), which the second replay
 * must sum. */
static void check_graph_replay(hipStream_t s)
{
    const int dt = AR_FP16, R = 2;
    const size_t n = 1000003, bytes = n * esize(dt);
    void *h[R], *d[R];
    for (int r = 0; r < R; ++r) {
        h[r] = host_values(dt, n, 3701 + r, 0.0, 1.0 / R);
        d[r] = to_device(h[r], bytes);
    }
    void *dout = to_device(NULL, bytes), *want = malloc(bytes);
    ar_params_t p = params(n, R, dt, d, dout);
    hipGraph_t g;
    hipGraphExec_t ge;
    CHECK_HIP(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
    const int32_t st = ar_sum(&p, s);
    CHECK_HIP(hipStreamEndCapture(s, &g));
    if (st != AR_OK)
        fail("ar_sum status under graph capture");
    CHECK_HIP(hipGraphInstantiate(&ge, g, NULL, NULL, 0));
    for (int round = 0; round < 2; ++round) {
        if (round == 1)
            for (int r = 0; r < R; ++r) {
                free(h[r]);
                h[r] = host_values(dt, n, 3801 + r, 0.0, 1.0 / R);
                CHECK_HIP(hipMemcpy(d[r], h[r], bytes, hipMemcpyHostToDevice));
            }
        CHECK_HIP(hipGraphLaunch(ge, s));
        CHECK_HIP(hipStreamSynchronize(s));
        void *got = from_device(dout, bytes);
        if (oracle_ar_sum(dt, R, (const void *const *)h, n, want) != 0)
            fail("oracle_ar_sum status (graph)");
        compare(round == 0 ? "fp16 sum from a HIP graph, first replay" : "fp16 sum from a HIP graph, second replay",
                dt, got, want, n, 1);
        free(got);
    }
    CHECK_HIP(hipGraphExecDestroy(ge));
    CHECK_HIP(hipGraphDestroy(g));
    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipFree(d[r]));
        free(h[r]);
    }
    CHECK_HIP(hipFree(dout));
    free(want);
}

static void check_host_calls(void)
{
    size_t offsets[AR_MAX_RANKS], total = 0;
    if (ar_partials_layout(1 << 20, AR_BF16, 4, offsets, &total) != AR_OK)
        fail("ar_partials_layout status");
    for (int r = 1; r < 4; ++r)
        if (offsets[r] < offsets[r - 1] + ((size_t)2 << 20) || offsets[r] % 256)
            fail("ar_partials_layout slots overlap or are misaligned");
    if (total < offsets[3] + ((size_t)2 << 20))
        fail("ar_partials_layout total too small");
}

int main(void)
{
    int devices = 0;
    CHECK_HIP(hipGetDeviceCount(&devices));
    if (devices < 1) {
        fprintf(stderr, "c_abi_check: no device\n");
        return 1;
    }
    CHECK_HIP(hipSetDevice(0));
    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    check_host_calls();
    check_sum(s);
    check_fused(s, AR_FP16, 4, 37, 640, 1, 0, "fp16 fused, 4 ranks, 37 x 640, bias and residual");
    check_fused(s, AR_FP32, 2, 9, 1024, 0, 1, "fp32 fused, 2 ranks, 9 x 1024, S over the residual");
    check_sum_slices(s);
    check_fused_slices(s);
    check_unfused(s);
    check_graph_replay(s);
    CHECK_HIP(hipStreamDestroy(s));
    if (failures)
        return 1;
    printf("c_abi_check: OK\n");
    return 0;
}
