/*
 * zf_oracle.c -- plain, sequential CPU oracle for the dominant-range exponent codec
 * (dense 3-bit planes plus sparse outlier records) of BF16 and FP8-E4M3FN tensors.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct definition against
 * which the HIP library's second codec is checked.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no source,
 * header, table or helper with the HIP library.  (It uses zxo_split from
 * zx_oracle.c, the other half of this oracle.)
 *
 * What is computed (ZipFloat page, "ZipFloat: An Ultra-fast and Lossless
 * Floating-Point Compressor for LLM Inference Systems"):
 *   - the tensor is cut into blocks of Ne = 2048 elements, each coded on its own
 *     (section 3.1);
 *   - per block, MD is the most frequent exponent, and the dominant range starts at
 *     l_b = MD - 6 with length L = 8 (section 3.2, Eq. 1-3 and the fixed values
 *     Delta* = 6, L* = 8 read off Fig. 3);
 *   - every exponent is remapped as new = old - l_b (section 3.2, Eq. 4), so that the
 *     dominant range lands on 0..7;
 *   - the low 3 bits of every remapped exponent go into a dense array packed as three
 *     bit planes of the block (768 bytes for 2048 elements), the remaining high bits
 *     are zero for in-range exponents and go, for the others, into 2-byte records of
 *     an 11-bit element index and a 5-bit field (section 3.3, dense and sparse
 *     packing);
 *   - sign and mantissa bits stay raw in a byte array (section 3.3, output assembly).
 *
 * Readings where the page leaves a step open (restated in the design notes):
 *   R1  ties for MD go to the smallest exponent value;
 *   R2  the subtraction of Eq. 4 is taken modulo the exponent field (2^8 for BF16,
 *       2^4 for FP8), so every exponent has a remapped value;
 *   R3  the 5-bit field of a record is the remapped exponent's bits 3..7 (the
 *       "sparse" part that is zero inside the dominant range); decoding ORs it above
 *       the dense bits;
 *   R4  plane p, byte k, bit i (least significant first) is bit p of element 8k+i's
 *       remapped exponent; a short last block pads with zero bits;
 *   R5  records are in increasing element order, and the records of all blocks are
 *       concatenated in block order, with u64 offsets from an exclusive prefix sum
 *       (the page reserves space with an atomic add; a prefix sum gives the same
 *       sizes and deterministic bytes);
 *   R6  FP8 uses the same rule with its 4-bit exponent: 3 dense bits and a 1-bit
 *       sparse part, in the same 2-byte record.
 *
 * Parity status: pinned by tests that do not reuse this code -- a hand-derived worked
 * block (tests/golden/zipfloat_block_example.txt), the exponent cost of Eq. 2
 * recomputed from a library histogram, MD against a library argmax, the record set
 * against a direct count of out-of-range exponents, and exhaustive round trips over
 * every BF16 and FP8 bit pattern.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ZFO_BF16 0
#define ZFO_FP8 1
#define ZFO_BLOCK 2048u           /* Ne, elements per block                         */
#define ZFO_PLANE_BYTES 256u      /* one bit per element of a block                 */
#define ZFO_DENSE_BITS 3u         /* ceil(log2 L*), L* = 8                          */
#define ZFO_DELTA 6               /* Delta* = MD - l_b                              */

#define ZFO_OK 0
#define ZFO_E_INVAL 1
#define ZFO_E_NOMEM 2
#define ZFO_E_CORRUPT 4

/* from zx_oracle.c: exponent field and sign+mantissa byte/nibble of each element */
void zxo_split(int dtype, const void *x, uint64_t n, uint8_t *exps, uint8_t *sm);

typedef struct zfo_container {
    int32_t dtype;
    int32_t reserved_;
    uint64_t n;
    uint64_t nblocks;          /* ceil(n / 2048)                                     */
    uint64_t nrecords;         /* total outlier records                              */
    uint64_t signmant_bytes;   /* n (BF16) or ceil(n / 2) (FP8)                      */
    uint8_t *lb;               /* [nblocks] start of the dominant range              */
    uint8_t *planes;           /* [nblocks][3][256]                                  */
    uint64_t *rec_off;         /* [nblocks + 1] record offsets                       */
    uint16_t *records;         /* [nrecords] (index << 5) | high bits                */
    uint8_t *signmant;         /* [signmant_bytes]                                   */
} zfo_container;

uint64_t zfo_sizeof_container(void) { return (uint64_t)sizeof(zfo_container); }

void zfo_free(zfo_container *c)
{
    free(c->lb);
    free(c->planes);
    free(c->rec_off);
    free(c->records);
    free(c->signmant);
    memset(c, 0, sizeof(*c));
}

static uint32_t field_of(int dtype) { return dtype == ZFO_BF16 ? 256u : 16u; }

/* Most frequent value of exps[0..m) over an alphabet of A symbols, ties to the
 * smallest (R1). */
uint32_t zfo_mode(const uint8_t *exps, uint64_t m, uint32_t A)
{
    uint64_t cnt[256];
    memset(cnt, 0, sizeof(cnt));
    for (uint64_t i = 0; i < m; ++i) cnt[exps[i]]++;
    uint32_t best = 0;
    for (uint32_t s = 1; s < A; ++s)
        if (cnt[s] > cnt[best]) best = s;
    return best;
}

int zfo_encode(int dtype, const void *x, uint64_t n, zfo_container *c)
{
    if (!c || (dtype != ZFO_BF16 && dtype != ZFO_FP8) || (n && !x)) return ZFO_E_INVAL;
    memset(c, 0, sizeof(*c));
    const uint32_t A = field_of(dtype);
    c->dtype = dtype;
    c->n = n;
    c->nblocks = (n + ZFO_BLOCK - 1) / ZFO_BLOCK;
    c->signmant_bytes = dtype == ZFO_BF16 ? n : (n + 1) / 2;
    uint8_t *exps = malloc(n ? n : 1);
    c->signmant = malloc(c->signmant_bytes ? c->signmant_bytes : 1);
    c->lb = malloc(c->nblocks ? c->nblocks : 1);
    c->planes = calloc(c->nblocks ? c->nblocks * ZFO_DENSE_BITS * ZFO_PLANE_BYTES : 1, 1);
    c->rec_off = calloc(c->nblocks + 1, sizeof(uint64_t));
    c->records = malloc((n ? n : 1) * sizeof(uint16_t));   /* at most one per element */
    if (!exps || !c->signmant || !c->lb || !c->planes || !c->rec_off || !c->records) {
        free(exps);
        zfo_free(c);
        return ZFO_E_NOMEM;
    }
    zxo_split(dtype, x, n, exps, c->signmant);
    uint64_t r = 0;
    for (uint64_t b = 0; b < c->nblocks; ++b) {
        const uint64_t lo = b * ZFO_BLOCK;
        const uint64_t m = (n - lo < ZFO_BLOCK) ? n - lo : ZFO_BLOCK;
        /* dominant range [l_b, l_b + 8) with l_b = MD - Delta* (mod the field, R2) */
        const uint32_t md = zfo_mode(exps + lo, m, A);
        const uint32_t lb = (md + A - ZFO_DELTA) % A;
        c->lb[b] = (uint8_t)lb;
        c->rec_off[b] = r;
        uint8_t *pl = c->planes + b * ZFO_DENSE_BITS * ZFO_PLANE_BYTES;
        for (uint64_t i = 0; i < m; ++i) {
            const uint32_t v = (exps[lo + i] + A - lb) % A;          /* Eq. 4 */
            for (uint32_t p = 0; p < ZFO_DENSE_BITS; ++p)            /* R4 */
                if ((v >> p) & 1u) pl[p * ZFO_PLANE_BYTES + i / 8] |= (uint8_t)(1u << (i % 8));
            const uint32_t high = v >> ZFO_DENSE_BITS;
            if (high) c->records[r++] = (uint16_t)((i << 5) | high);   /* R3, R5 */
        }
    }
    c->rec_off[c->nblocks] = r;
    c->nrecords = r;
    free(exps);
    return ZFO_OK;
}

int zfo_decode(const zfo_container *c, void *out)
{
    if (!c || (c->dtype != ZFO_BF16 && c->dtype != ZFO_FP8) || (c->n && !out)) return ZFO_E_INVAL;
    const uint32_t A = field_of(c->dtype);
    for (uint64_t b = 0; b < c->nblocks; ++b) {
        const uint64_t lo = b * ZFO_BLOCK;
        const uint64_t m = (c->n - lo < ZFO_BLOCK) ? c->n - lo : ZFO_BLOCK;
        const uint8_t *pl = c->planes + b * ZFO_DENSE_BITS * ZFO_PLANE_BYTES;
        uint8_t high[ZFO_BLOCK];
        memset(high, 0, sizeof(high));
        if (c->rec_off[b] > c->rec_off[b + 1] || c->rec_off[b + 1] > c->nrecords) return ZFO_E_CORRUPT;
        for (uint64_t k = c->rec_off[b]; k < c->rec_off[b + 1]; ++k) {
            const uint32_t idx = c->records[k] >> 5;
            if (idx >= m) return ZFO_E_CORRUPT;
            high[idx] = (uint8_t)(c->records[k] & 31u);
        }
        for (uint64_t i = 0; i < m; ++i) {
            uint32_t v = (uint32_t)high[i] << ZFO_DENSE_BITS;
            for (uint32_t p = 0; p < ZFO_DENSE_BITS; ++p) v |= ((pl[p * ZFO_PLANE_BYTES + i / 8] >> (i % 8)) & 1u) << p;
            const uint32_t e = (v + c->lb[b]) % A;                     /* inverse of Eq. 4 */
            const uint64_t j = lo + i;
            if (c->dtype == ZFO_BF16) {
                const uint32_t sm = c->signmant[j];
                ((uint16_t *)out)[j] = (uint16_t)(((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu));
            } else {
                const uint32_t nib = (c->signmant[j / 2] >> (4 * (j % 2))) & 0xFu;
                ((uint8_t *)out)[j] = (uint8_t)(((nib & 0x8u) << 4) | (e << 3) | (nib & 0x7u));
            }
        }
    }
    return ZFO_OK;
}
