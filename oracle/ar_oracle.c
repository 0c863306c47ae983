/*
 * CPU oracle for the all-reduce core: the rank-partial sum, and the sum fused
 * with GEMM bias, residual and RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against. Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it. It shares no
 * code, header, table or constant with the GPU library and includes nothing
 * from it.
 *
 * Sources (the pages this follows):
 *   [AR-Plugin]  "All Reduce Plugin" (TensorRT-Edge-LLM C++ API),
 *                class AllReducePlugin description: the op is an all-reduce
 *                SUM of the partial activations that tensor-parallel ranks
 *                produce after a row-parallel linear; with one rank it is a
 *                passthrough.
 *   [type.d2]    "type.d2", class AllReduceParams (elts_total, the per-rank
 *                buffer array, the output buffer) and class
 *                AllReduceFusionParams (bias_buffer = the GEMM bias,
 *                residual_buffer, the RMSNorm fields hidden_size,
 *                weight_buffer, eps, and intermediate_buffer);
 *                enum AllReduceFusionOp {NONE, RESIDUAL_RMS_NORM}.
 *   [allreduce.d2] "allreduce.d2", kernels customAllReduceKernels.cu:
 *                the standalone branch (oneShotAllReduceKernel), the fused
 *                branch (one_shot_all_reduce_norm_kernel -> rms_norm) and the
 *                unfused branch (twoShotAllReduceKernel then rms_norm_kernel).
 *
 * Readings taken where the pages are silent (every one is listed in the
 * design notes of this repository):
 *   - the rank sum accumulates in fp32, in rank index order 0..R-1, starting
 *     from the value of rank 0 (not from +0.0);
 *   - the bias is a [hidden] vector added once, after the rank sum, then the
 *     residual is added; that fp32 value is rounded once to the element type
 *     and stored as the pre-norm sum S (intermediate_buffer);
 *   - RMSNorm runs on the ROUNDED S:  y = S / sqrt(mean_h(S^2) + eps) * W,
 *     with divisor hidden_size, eps inside the square root, no mean
 *     subtraction and no shift term;
 *   - the norm is computed in fp64 here and rounded once to the element type;
 *   - fp16/bf16 rounding is IEEE round-to-nearest-even, overflow to +-Inf,
 *     NaN stays NaN (payload not meaningful), subnormals kept.
 *
 * Built with: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 * (no fused multiply-add, no reassociation; on x86-64 float arithmetic is
 * done in SSE single precision, so each fp32 add rounds once).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* Element-type codes of this oracle (its own numbering). */
#define ORC_FP32 0
#define ORC_FP16 1
#define ORC_BF16 2

/* ----------------------------------------------------------------------
 * Binary floating-point formats, written from the IEEE 754 definition of
 * a binary format with p significand bits (p-1 stored), exponent bias
 * `bias` and all-ones exponent for Inf/NaN.
 *   binary16 (fp16): 1 sign, 5 exponent, 10 fraction bits, bias 15
 *   bfloat16 (bf16): 1 sign, 8 exponent,  7 fraction bits, bias 127
 * -------------------------------------------------------------------- */
typedef struct {
    int frac_bits; /* stored fraction bits          */
    int exp_bits;  /* exponent field width          */
    int bias;      /* exponent bias                 */
} orc_format;

static const orc_format ORC_FMT_F16 = {10, 5, 15};
static const orc_format ORC_FMT_BF16 = {7, 8, 127};

/* Value of a 16-bit encoding. */
static double orc_decode16(uint16_t bits, orc_format f)
{
    int sign = (bits >> 15) & 1;
    int emax_field = (1 << f.exp_bits) - 1;
    int e = (bits >> f.frac_bits) & emax_field;
    uint32_t m = bits & ((1u << f.frac_bits) - 1u);
    double v;
    if (e == emax_field) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        /* subnormal: m * 2^(1 - bias - frac_bits) */
        v = ldexp((double)m, 1 - f.bias - f.frac_bits);
    } else {
        /* normal: (2^frac_bits + m) * 2^(e - bias - frac_bits) */
        v = ldexp((double)((1u << f.frac_bits) + m), e - f.bias - f.frac_bits);
    }
    return sign ? -v : v;
}

/*
 * Nearest 16-bit encoding of x, ties to even significand.
 * The spacing of representable numbers ("quantum") in the binade of x is
 * 2^(E - frac_bits), where E = floor(log2|x|), and it is 2^(1-bias-frac_bits)
 * for every |x| below the smallest normal. x / quantum is exact in double (a
 * power-of-two scaling), and nearbyint() rounds it half-to-even in the
 * default rounding mode. With q = that rounded integer:
 *   subnormal range: the encoding is q itself (q == 2^frac_bits is then the
 *                    smallest normal, which that same integer encodes);
 *   normal range:    encoding = (E + bias) << frac_bits  +  (q - 2^frac_bits);
 *                    q == 2^(frac_bits+1) (a carry out of the binade) then
 *                    lands on the next exponent with zero fraction, and
 *                    carrying past the largest exponent gives Inf.
 */
static uint16_t orc_encode16(double x, orc_format f)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    int emax_field = (1 << f.exp_bits) - 1;
    uint16_t inf_bits = (uint16_t)(emax_field << f.frac_bits);
    if (isnan(x))
        return (uint16_t)(sign | inf_bits | (1u << (f.frac_bits - 1))); /* quiet NaN */
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | inf_bits);
    if (a == 0.0)
        return sign;

    int emin = 1 - f.bias;               /* exponent of the smallest normal */
    int emax = emax_field - 1 - f.bias;  /* exponent of the largest finite  */
    int fe;
    (void)frexp(a, &fe);                 /* a = m * 2^fe, m in [0.5, 1)     */
    int E = fe - 1;                      /* a in [2^E, 2^(E+1))             */
    if (E > emax)
        return (uint16_t)(sign | inf_bits);

    if (E < emin) {
        double q = nearbyint(ldexp(a, f.bias - 1 + f.frac_bits)); /* a / 2^(emin - frac_bits) */
        return (uint16_t)(sign | (uint16_t)q);
    }
    double q = nearbyint(ldexp(a, f.frac_bits - E));              /* a / 2^(E - frac_bits)    */
    uint32_t bits = ((uint32_t)(E + f.bias) << f.frac_bits) + ((uint32_t)q - (1u << f.frac_bits));
    if (bits > inf_bits)
        bits = inf_bits;
    return (uint16_t)(sign | bits);
}

/* Exported converters (pinned by the tests against numpy/torch). */
double oracle_f64_from_f16(uint16_t h) { return orc_decode16(h, ORC_FMT_F16); }
double oracle_f64_from_bf16(uint16_t h) { return orc_decode16(h, ORC_FMT_BF16); }
uint16_t oracle_f16_from_f64(double x) { return orc_encode16(x, ORC_FMT_F16); }
uint16_t oracle_bf16_from_f64(double x) { return orc_encode16(x, ORC_FMT_BF16); }

static size_t orc_elem_size(int dtype)
{
    return dtype == ORC_FP32 ? 4u : 2u;
}

/* Element i of a buffer of the given type, widened to fp32. Widening an
 * fp16 or bf16 value to fp32 is exact. */
static float orc_load(int dtype, const void *buf, size_t i)
{
    if (dtype == ORC_FP32) {
        float v;
        memcpy(&v, (const char *)buf + 4 * i, 4);
        return v;
    }
    uint16_t h;
    memcpy(&h, (const char *)buf + 2 * i, 2);
    return (float)(dtype == ORC_FP16 ? oracle_f64_from_f16(h) : oracle_f64_from_bf16(h));
}

/* Store x rounded (once, to nearest even) to the element type. */
static void orc_store(int dtype, void *buf, size_t i, double x)
{
    if (dtype == ORC_FP32) {
        float v = (float)x; /* C conversion double -> float: current rounding mode (nearest even) */
        memcpy((char *)buf + 4 * i, &v, 4);
        return;
    }
    uint16_t h = dtype == ORC_FP16 ? oracle_f16_from_f64(x) : oracle_bf16_from_f64(x);
    memcpy((char *)buf + 2 * i, &h, 2);
}

static int orc_check(int dtype, int ranks, const void *const *parts)
{
    if (dtype != ORC_FP32 && dtype != ORC_FP16 && dtype != ORC_BF16)
        return -1;
    if (ranks < 1 || !parts)
        return -1;
    for (int r = 0; r < ranks; ++r)
        if (!parts[r])
            return -1;
    return 0;
}

/* fp32 sum of the R partials at element i: start at rank 0, add ranks
 * 1..R-1 in index order, one rounding per add. [AR-Plugin] (sum), [type.d2]
 * (per-rank buffers indexed by rank). */
static float orc_rank_sum(int dtype, int ranks, const void *const *parts, size_t i)
{
    float a = orc_load(dtype, parts[0], i);
    for (int r = 1; r < ranks; ++r)
        a = a + orc_load(dtype, parts[r], i);
    return a;
}

/*
 * Fusion op NONE ([type.d2] enum AllReduceFusionOp; [allreduce.d2]
 * standalone branch): out[i] = round_T( sum_r parts[r][i] ), i < n.
 * out may be the same buffer as one of the partials.
 */
int oracle_ar_sum(int dtype, int ranks, const void *const *parts, size_t n, void *out)
{
    if (orc_check(dtype, ranks, parts) || (n && !out))
        return -1;
    for (size_t i = 0; i < n; ++i)
        orc_store(dtype, out, i, (double)orc_rank_sum(dtype, ranks, parts, i));
    return 0;
}

/*
 * RMSNorm of each row of x ([rows, hidden], rows = n / hidden), as the
 * rms_norm step of [allreduce.d2] with the RMSNorm fields of [type.d2]
 * AllReduceFusionParams (hidden_size, weight_buffer, eps):
 *   ms    = (1/hidden) * sum_h x[t,h]^2          (fp64, h in order)
 *   rstd  = 1 / sqrt(ms + eps)                   (fp64)
 *   out[t,h] = round_T( x[t,h] * rstd * w[h] )   (fp64, then one rounding)
 * out may be the same buffer as x.
 */
int oracle_rmsnorm(int dtype, size_t n, int hidden, const void *x, const void *weight, float eps, void *out)
{
    if (dtype != ORC_FP32 && dtype != ORC_FP16 && dtype != ORC_BF16)
        return -1;
    if (hidden <= 0 || n % (size_t)hidden)
        return -1;
    if (n && (!x || !weight || !out))
        return -1;
    size_t rows = n / (size_t)hidden;
    for (size_t t = 0; t < rows; ++t) {
        size_t row = t * (size_t)hidden;
        double ss = 0.0;
        for (int h = 0; h < hidden; ++h) {
            double s = (double)orc_load(dtype, x, row + (size_t)h);
            ss = ss + s * s;
        }
        double rstd = 1.0 / sqrt(ss / (double)hidden + (double)eps);
        for (int h = 0; h < hidden; ++h) {
            double s = (double)orc_load(dtype, x, row + (size_t)h);
            double w = (double)orc_load(dtype, weight, (size_t)h);
            orc_store(dtype, out, row + (size_t)h, s * rstd * w);
        }
    }
    return 0;
}

/*
 * Fusion op RESIDUAL_RMS_NORM ([type.d2] AllReduceFusionParams; [allreduce.d2]
 * one_shot_all_reduce_norm_kernel -> rms_norm):
 *   a        = sum_r parts[r][i]            (fp32, rank order)
 *   a        = a + bias[h]                  (if bias;     fp32)
 *   a        = a + residual[i]              (if residual; fp32)
 *   S[i]     = round_T(a)  -> intermediate[i]
 *   out      = RMSNorm(S) over each row of `hidden` elements (oracle_rmsnorm)
 * with i = t*hidden + h. NULL bias or residual means that add is skipped.
 * intermediate may be the residual buffer; out may be one of the partials.
 */
int oracle_ar_residual_rmsnorm(int dtype, int ranks, const void *const *parts, size_t n, int hidden,
                               const void *bias, const void *residual, const void *weight, float eps,
                               void *out, void *intermediate)
{
    if (orc_check(dtype, ranks, parts))
        return -1;
    if (hidden <= 0 || n % (size_t)hidden)
        return -1;
    if (n && (!weight || !out || !intermediate))
        return -1;
    for (size_t i = 0; i < n; ++i) {
        float a = orc_rank_sum(dtype, ranks, parts, i);
        if (bias)
            a = a + orc_load(dtype, bias, i % (size_t)hidden);
        if (residual)
            a = a + orc_load(dtype, residual, i);
        orc_store(dtype, intermediate, i, (double)a);
    }
    return oracle_rmsnorm(dtype, n, hidden, intermediate, weight, eps, out);
}

size_t oracle_elem_size(int dtype) { return orc_elem_size(dtype); }
