/*
 * oracle.c -- plain, slow, scalar CPU oracle for one rank's ZeRO shard step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or constant with the HIP
 * library: it has its own binary16 codec, its own layout and ledger
 * arithmetic and its own Adam.
 *
 * Sources (the three web pages this library is built from):
 *   [16B]  "Your 7.5B model's weights fit in 15 GB ... the 16-byte parameter
 *          and ZeRO's three-stage split" (blog.teqners.com)
 *   [ER10] "ZeRO and the Memory Tricks", The Engine Room ch. 10
 *          (hoshank.vercel.app)
 *   [DSZ]  "DeepSpeed ZeRO: account for every training state"
 *          (chenhuiyu.github.io)
 *
 * Precision: the pages fix the state precisions (fp16 parameter and gradient,
 * fp32 master, momentum and variance: [16B] "Where 16 bytes per parameter
 * comes from", state table; [ER10] "The Mathematics", ledger table) and say
 * the optimizer state is kept and updated in fp32 ([16B] "Why you can't just
 * delete the fp32 copies").  So every Adam operation below is one IEEE-754
 * binary32 operation with round-to-nearest-even, in the order written, with
 * no fused multiply-add (built with -ffp-contract=off, SSE scalar math, no
 * excess precision).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math
 *        -fno-tree-vectorize -fPIC -shared oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_EOVERFLOW (-2)

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32.                                           */
/* [16B] "Where 16 bytes per parameter comes from" (fp16 rows of the state  */
/* table) and "Why you can't just delete the fp32 copies" (underflow below  */
/* 2^-24).  binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction    */
/* bits.  A normal value is (1 + F/1024) * 2^(E-15) for E in 1..30; a       */
/* subnormal (E = 0) is F * 2^-24; E = 31 is infinity (F = 0) or NaN.       */
/* ------------------------------------------------------------------------ */

float orc_f16_to_f32(uint16_t h)
{
    int negative = (h >> 15) & 1;
    int E = (h >> 10) & 0x1f;
    int F = h & 0x3ff;
    double mag;
    if (E == 0) {
        mag = ldexp((double)F, -24);
    } else if (E == 31) {
        if (F != 0)
            return negative ? -NAN : NAN;
        mag = INFINITY;
    } else {
        mag = ldexp(1024.0 + (double)F, E - 25);
    }
    return (float)(negative ? -mag : mag); /* exact: every binary16 fits */
}

/*
 * Round a binary32 value to the nearest binary16 value, ties to the one with
 * an even last fraction bit.  The quantum (spacing of binary16 values) at a
 * magnitude a in [2^(e-1), 2^e) is 2^(e-11) for normal numbers and 2^-24 for
 * the subnormal range, so the rounded magnitude is rint(a / quantum) *
 * quantum, with rint rounding half to even (the default rounding mode).  The
 * division is a power-of-two scaling of a double and therefore exact.
 * Magnitudes from 65520 up (halfway between the largest finite value 65504 and
 * 2^16, which ties to the even neighbour 2^16) overflow to infinity.
 */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7e00; /* a quiet NaN; the payload is not kept */
    double a = fabs((double)x);
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e); /* a = f * 2^e with 0.5 <= f < 1 */
    int q = e - 11;
    if (q < -24)
        q = -24;
    double k = nearbyint(ldexp(a, -q)); /* number of quanta, ties to even */
    double r = ldexp(k, q);              /* the rounded magnitude */
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -14)) /* subnormal: F quanta of 2^-24 */
        return sign | (uint16_t)ldexp(r, 24);
    int er;
    double fr = frexp(r, &er);  /* r = fr * 2^er, r may have carried up */
    int E = er - 1 + 15;        /* r = (2 fr) * 2^(er-1), 1 <= 2 fr < 2 */
    int F = (int)((2.0 * fr - 1.0) * 1024.0);
    return sign | (uint16_t)(E << 10) | (uint16_t)F;
}

void orc_f32_to_f16_array(const float *x, uint16_t *out, uint64_t n)
{
    for (uint64_t i = 0; i < n; i++)
        out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_array(const uint16_t *h, float *out, uint64_t n)
{
    for (uint64_t i = 0; i < n; i++)
        out[i] = orc_f16_to_f32(h[i]);
}

static int orc_f16_is_finite(uint16_t h)
{
    return ((h >> 10) & 0x1f) != 31;
}

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> binary32.                                                    */
/* [DSZ] "Why parameter count is not training memory": BF16 setups differ   */
/* in which states they keep; this variant keeps the 16-byte ledger with    */
/* bfloat16 parameters and gradients in place of fp16.  bfloat16: 1 sign    */
/* bit, binary32's 8 exponent bits (bias 127) and 7 fraction bits.  A       */
/* normal value is (1 + F/128) * 2^(E-127) for E in 1..254; a subnormal     */
/* (E = 0) is F * 2^-133; E = 255 is infinity (F = 0) or NaN.               */
/* ------------------------------------------------------------------------ */
float orc_bf16_to_f32(uint16_t h)
{
    int negative = (h >> 15) & 1;
    int E = (h >> 7) & 0xff;
    int F = h & 0x7f;
    double mag;
    if (E == 0) {
        mag = ldexp((double)F, -133);
    } else if (E == 255) {
        if (F != 0)
            return negative ? -NAN : NAN;
        mag = INFINITY;
    } else {
        mag = ldexp(128.0 + (double)F, E - 134);
    }
    return (float)(negative ? -mag : mag); /* exact: every bfloat16 fits */
}

/*
 * Round a binary32 value to the nearest bfloat16 value, ties to the one with
 * an even last fraction bit.  The quantum at a magnitude a in [2^(e-1), 2^e)
 * is 2^(e-8) for normal numbers and 2^-133 in the subnormal range; the
 * rounded magnitude is rint(a / quantum) * quantum (rint: half to even).
 * Magnitudes from (2 - 2^-8) * 2^127 up (halfway between the largest finite
 * value (2 - 2^-7) * 2^127 and 2^128, a tie that goes to the even 2^128)
 * overflow to infinity.
 */
uint16_t orc_f32_to_bf16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return sign | 0x7fc0; /* a quiet NaN; the payload is not kept */
    double a = fabs((double)x);
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))
        return sign | 0x7f80;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int q = e - 8;
    if (q < -133)
        q = -133;
    double quanta = nearbyint(ldexp(a, -q)); /* ties to even */
    double r = ldexp(quanta, q);
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -126)) /* subnormal: F quanta of 2^-133 */
        return sign | (uint16_t)ldexp(r, 133);
    int er;
    double fr = frexp(r, &er);
    int E = er - 1 + 127;
    int F = (int)((2.0 * fr - 1.0) * 128.0);
    return sign | (uint16_t)(E << 7) | (uint16_t)F;
}

void orc_f32_to_bf16_array(const float *x, uint16_t *out, uint64_t n)
{
    for (uint64_t i = 0; i < n; i++)
        out[i] = orc_f32_to_bf16(x[i]);
}

void orc_bf16_to_f32_array(const uint16_t *h, float *out, uint64_t n)
{
    for (uint64_t i = 0; i < n; i++)
        out[i] = orc_bf16_to_f32(h[i]);
}

/* The two 16-bit formats of the parameters and gradients. */
#define ORC_FMT_F16 0
#define ORC_FMT_BF16 1

static float orc_widen(int fmt, uint16_t h)
{
    return fmt == ORC_FMT_BF16 ? orc_bf16_to_f32(h) : orc_f16_to_f32(h);
}

static uint16_t orc_narrow(int fmt, float x)
{
    return fmt == ORC_FMT_BF16 ? orc_f32_to_bf16(x) : orc_f32_to_f16(x);
}

static int orc_is_finite(int fmt, uint16_t h)
{
    return fmt == ORC_FMT_BF16 ? ((h >> 7) & 0xff) != 255 : orc_f16_is_finite(h);
}

/* ------------------------------------------------------------------------ */
/* Shard layout of the flat buffer.                                          */
/* Each of the N_d ranks owns one contiguous slice of the flattened state    */
/* ([16B] "The replication nobody questioned", "The part that sounds too     */
/* good: communication"; [DSZ] "ZeRO removes replicated state in stages").   */
/* The pages fix no padding rule; the flat buffer is padded at its tail to a  */
/* multiple of N_d * align elements so all shards have the same length,      */
/* a multiple of align, and the padding lands in the last shards.            */
/* out = {padded_total, shard_len, offset, real_len}                         */
/* ------------------------------------------------------------------------ */
int orc_shard_layout(uint64_t psi, uint32_t nd, uint32_t rank, uint32_t align,
                     uint64_t out[4])
{
    if (nd == 0 || align == 0 || rank >= nd)
        return ORC_EINVAL;
    unsigned __int128 unit = (unsigned __int128)nd * align;
    unsigned __int128 units = ((unsigned __int128)psi + unit - 1) / unit;
    unsigned __int128 padded = units * unit;
    if (padded > UINT64_MAX)
        return ORC_EOVERFLOW;
    uint64_t shard = (uint64_t)(padded / nd);
    uint64_t offset = (uint64_t)rank * shard;
    uint64_t real = 0;
    if (offset < psi)
        real = (psi - offset < shard) ? psi - offset : shard;
    out[0] = (uint64_t)padded;
    out[1] = shard;
    out[2] = offset;
    out[3] = real;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Model-state ledger, bytes resident on one rank.                           */
/* [ER10] "The Mathematics", eq. M_states = (2 + 2 + K) Psi with K = 12 and  */
/* eq. M_states(p, N_d); [16B] "The replication nobody questioned", stage    */
/* table; [DSZ] "ZeRO removes replicated state in stages".                   */
/*   stage 0 (plain data parallel): 16 Psi                                   */
/*   stage 1: 4 Psi + 12 S     stage 2: 2 Psi + 14 S     stage 3: 16 S       */
/* where S is the padded shard length, the pages' Psi / N_d.                 */
/* ------------------------------------------------------------------------ */
int orc_state_bytes(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t align,
                    uint64_t *out)
{
    if (stage > 3)
        return ORC_EINVAL;
    uint64_t lay[4];
    int rc = orc_shard_layout(psi, nd, 0, align, lay);
    if (rc != ORC_OK)
        return rc;
    unsigned __int128 P = psi, S = lay[1], b;
    switch (stage) {
    case 0: b = 16 * P; break;
    case 1: b = 4 * P + 12 * S; break;
    case 2: b = 2 * P + 14 * S; break;
    default: b = 16 * S; break;
    }
    if (b > UINT64_MAX)
        return ORC_EOVERFLOW;
    *out = (uint64_t)b;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Adam (Kingma and Ba, Algorithm 1, with bias correction, epsilon outside   */
/* the square root).  The pages name Adam's first and second moments and     */
/* the fp32 master copy ([ER10] "Where We Were", "The Mathematics" ledger    */
/* table; [16B] "Where 16 bytes per parameter comes from") but print no      */
/* update equations, so the textbook algorithm is used.                      */
/*                                                                           */
/* hp = {lr, beta1, beta2, eps, weight_decay}; t >= 1 is the 1-based step.   */
/* Scalars are formed in double and rounded to binary32 once each:           */
/*   out = {lr, b1, 1-b1, b2, 1-b2, 1-b1^t, 1-b2^t, eps}                     */
/* Weight decay is not defined by the pages and must be 0.                   */
/* ------------------------------------------------------------------------ */
int orc_adam_scalars(const double hp[5], uint64_t t, float out[8])
{
    if (t == 0 || hp[4] != 0.0)
        return ORC_EINVAL;
    double b1 = hp[1], b2 = hp[2];
    out[0] = (float)hp[0];
    out[1] = (float)b1;
    out[2] = (float)(1.0 - b1);
    out[3] = (float)b2;
    out[4] = (float)(1.0 - b2);
    out[5] = (float)(1.0 - pow(b1, (double)t));
    out[6] = (float)(1.0 - pow(b2, (double)t));
    out[7] = (float)hp[3];
    return ORC_OK;
}

/*
 * One Adam step over n elements of this rank's shard.  Per element:
 *   g  = fp32(grad16)
 *   m  = b1 m + (1-b1) g
 *   v  = b2 v + (1-b2) g^2
 *   mh = m / (1-b1^t)           vh = v / (1-b2^t)
 *   w  = w - lr * mh / (sqrt(vh) + eps)
 *   param16 = round-to-nearest-even binary16 of w
 * The master copy w, m and v are updated in place and the fp16 parameter is
 * written fresh from the updated master ([16B] "Why you can't just delete the
 * fp32 copies": updates accumulate in the fp32 master, the fp16 weights are
 * derived from it).  Non-finite values follow IEEE arithmetic element by
 * element.  Returns 1 if any gradient (after the loss scale's 2^-k, in the
 * scaled step) is infinite or NaN, else 0; if skip is nonzero nothing is
 * read or written and 0 is returned.
 */
static int adam_over(int fmt, uint64_t n, const uint16_t *grad16, uint16_t *param16,
                     float *w, float *m, float *v, const double hp[5], uint64_t t,
                     int skip, int scaled, float unscale)
{
    if (fmt != ORC_FMT_F16 && fmt != ORC_FMT_BF16)
        return ORC_EINVAL;
    float s[8];
    int rc = orc_adam_scalars(hp, t, s);
    if (rc != ORC_OK)
        return rc;
    if (skip)
        return 0;
    const float lr = s[0], b1 = s[1], omb1 = s[2], b2 = s[3], omb2 = s[4];
    const float bc1 = s[5], bc2 = s[6], eps = s[7];
    int flag = 0;
    for (uint64_t i = 0; i < n; i++) {
        float g = orc_widen(fmt, grad16[i]);
        if (scaled)
            g = g * unscale;
        /* the flag looks at the gradient the update uses: infinite or NaN
           when the 16-bit value is, or when 2^-k carries a finite bfloat16
           value past the fp32 range (k < 0) */
        if (!isfinite(g))
            flag = 1;

        float m_old = b1 * m[i];
        float m_in = omb1 * g;
        float m_new = m_old + m_in;

        float v_old = b2 * v[i];
        float g2 = g * g;
        float v_in = omb2 * g2;
        float v_new = v_old + v_in;

        float m_hat = m_new / bc1;
        float v_hat = v_new / bc2;
        float root = sqrtf(v_hat);
        float denom = root + eps;
        float u = m_hat / denom;
        float step = lr * u;
        float w_new = w[i] - step;

        m[i] = m_new;
        v[i] = v_new;
        w[i] = w_new;
        param16[i] = orc_narrow(fmt, w_new);
    }
    return flag;
}

int orc_adam_step_fmt(int fmt, uint64_t n, const uint16_t *grad16, uint16_t *param16,
                      float *w, float *m, float *v, const double hp[5], uint64_t t,
                      int skip)
{
    return adam_over(fmt, n, grad16, param16, w, m, v, hp, t, skip, 0, 1.0f);
}

/*
 * The same step on gradients that carry a loss scale of 2^k.  The pages do
 * not treat loss scaling; they do say that fp16 loses gradient values below
 * 2^-24 ([16B] "Why you can't just delete the fp32 copies"), which is what a
 * scale on the loss, and so on every gradient, works against.  Reading: the
 * widened gradient is multiplied by 2^-k in fp32 before the update above.
 * For fp16 and |k| <= 100 this product is exact for every finite value (it
 * stays a normal fp32 number), so the step equals the unscaled step on the
 * true gradient whenever that gradient is itself an fp16 value.  bfloat16
 * has the fp32 exponent range: there the product is exact only while it
 * stays a normal fp32 number (k > 0 can push small values into the
 * subnormals or to zero, k < 0 large ones to infinity, which raises the
 * flag).  Other k are rejected.
 */
int orc_adam_step_scaled(int fmt, uint64_t n, const uint16_t *grad16, uint16_t *param16,
                         float *w, float *m, float *v, const double hp[5], uint64_t t,
                         int32_t log2_scale, int skip)
{
    if (log2_scale < -100 || log2_scale > 100)
        return ORC_EINVAL;
    const float unscale = (float)ldexp(1.0, -log2_scale);
    return adam_over(fmt, n, grad16, param16, w, m, v, hp, t, skip, 1, unscale);
}

/* The fp16 step above (the pages' 16-byte ledger). */
int orc_adam_step(uint64_t n, const uint16_t *grad16, uint16_t *param16,
                  float *w, float *m, float *v, const double hp[5], uint64_t t,
                  int skip)
{
    return orc_adam_step_fmt(ORC_FMT_F16, n, grad16, param16, w, m, v, hp, t, skip);
}

/* ------------------------------------------------------------------------ */
/* Gradient reduction for this rank's partition.                             */
/* After the reduce-scatter, a rank holds the summed gradient of its own    */
/* partition only ([16B] "The part that sounds too good: communication";     */
/* [ER10] "The Mathematics", communication paragraph).  Here the N_d ranks'  */
/* fp16 slices of this partition are given as N_d arrays.  The pages do not  */
/* fix order, precision or scaling; this oracle sums in fp32 in rank order   */
/* (the first slice initialises the sum), divides once by N_d, and rounds    */
/* to fp16 (the stage-2 ledger keeps 2 bytes of gradient per parameter).     */
/* Returns 1 if any output is infinite or NaN, else 0.                       */
/* ------------------------------------------------------------------------ */
int orc_reduce_fmt(int fmt, uint32_t nd, const uint16_t *const *slices, uint64_t n,
                   uint16_t *out)
{
    if (nd == 0 || (fmt != ORC_FMT_F16 && fmt != ORC_FMT_BF16))
        return ORC_EINVAL;
    const float count = (float)nd;
    int flag = 0;
    for (uint64_t i = 0; i < n; i++) {
        float acc = orc_widen(fmt, slices[0][i]);
        for (uint32_t r = 1; r < nd; r++)
            acc = acc + orc_widen(fmt, slices[r][i]);
        float mean = acc / count;
        out[i] = orc_narrow(fmt, mean);
        if (!orc_is_finite(fmt, out[i]))
            flag = 1;
    }
    return flag;
}

/* The fp16 reduction (the pages' 2-byte gradients). */
int orc_reduce(uint32_t nd, const uint16_t *const *slices, uint64_t n,
               uint16_t *out)
{
    return orc_reduce_fmt(ORC_FMT_F16, nd, slices, n, out);
}

/* ------------------------------------------------------------------------ */
/* Communication volume of one training step, per rank.                      */
/* [16B] "The part that sounds too good: communication"; [ER10] "The         */
/* Mathematics", communication paragraph, and "What It Enabled", stage      */
/* table.  Plain data parallelism (stage 0) all-reduces, which in a ring   */
/* takes two passes of Psi each (reduce-scatter, then all-gather): 2 Psi per */
/* step.  Stages 1 and 2 reduce-scatter the gradients (Psi) and gather the  */
/* fresh fp16 parameter shards to every rank (Psi): 2 Psi.  Stage 3 also     */
/* all-gathers the parameters on demand in the forward and in the backward   */
/* pass, besides the gradient reduce-scatter: 3 Psi, 1.5x.  Volumes count    */
/* elements (the pages' multiples of Psi); with fp16 gradients and          */
/* parameters each is 2 bytes.                                               */
/* out = {passes, volume = passes * Psi, ring_send = passes * (nd - 1) * S}  */
/* where one ring pass over the padded layout has every rank send nd - 1     */
/* shards of S elements to its neighbour.                                    */
/* ------------------------------------------------------------------------ */
int orc_comm_volume(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t align,
                    uint64_t out[3])
{
    if (stage > 3)
        return ORC_EINVAL;
    uint64_t lay[4];
    int rc = orc_shard_layout(psi, nd, 0, align, lay);
    if (rc != ORC_OK)
        return rc;
    uint64_t passes = stage == 3 ? 3 : 2;
    unsigned __int128 volume = (unsigned __int128)passes * psi;
    unsigned __int128 ring = (unsigned __int128)passes * (nd - 1) * lay[1];
    if (volume > UINT64_MAX || ring > UINT64_MAX)
        return ORC_EOVERFLOW;
    out[0] = passes;
    out[1] = (uint64_t)volume;
    out[2] = (uint64_t)ring;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Receive side of the parameter all-gather: after it, every rank holds the */
/* whole fp16 parameter buffer, rank r's updated shard at r * S ([16B] "The  */
/* part that sounds too good: communication").  Here the N_d shards are     */
/* given as N_d arrays of S elements: full[r * S + i] = shards[r][i].        */
/* ------------------------------------------------------------------------ */
int orc_gather(uint32_t nd, const uint16_t *const *shards, uint64_t shard_len,
               uint16_t *full)
{
    if (nd == 0)
        return ORC_EINVAL;
    for (uint32_t r = 0; r < nd; r++)
        for (uint64_t i = 0; i < shard_len; i++)
            full[(uint64_t)r * shard_len + i] = shards[r][i];
    return ORC_OK;
}
