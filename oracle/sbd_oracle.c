/*
 * sbd_oracle.c -- the CPU oracle for the bf16 delta-sync hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no header, helper, table or constant
 * with the HIP path.
 *
 * Every routine is the plain definition, written as single-threaded uint16
 * loops over bf16 bit patterns, in the order the sources describe.  No
 * blocking, no vectorisation, no reordering.
 *
 * Sources (page titles; the pages are web articles, cited by section):
 *  [TRL]   "Shipping a Trillion Parameters With a Hub Bucket: Delta Weight Sync
 *          in TRL" (Hugging Face blog; Korean translation and a Chinese summary).
 *  [VERL]  verl PR #6974 review, "delta_sharded" checkpoint engine (prhub).
 *  [XOR]   humans& "weight sync in RL with under 0.23 s pause" (news summary).
 *
 * Pinning (how each routine is checked against something other than itself)
 * is listed beside each function; the tests live in tests/test_oracle.py.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

#define ORACLE_INT32_MAX 2147483647LL

/*
 * oracle_diff -- bitwise change detection plus stream compaction.
 *
 * [VERL] code-snippet section, sparse_gather.py `shard_delta_indices`: the two
 * snapshots are reinterpreted as same-width integers, compared with `!=`, and
 * the positions of the differing elements are taken in ascending order
 * (`nonzero`), with the new values gathered at those positions.
 * [TRL] section 4.1 (safetensors as the wire format): per changed parameter a
 * flat int32 tensor of element indices and a bf16 tensor of the values at
 * those indices.
 *
 * Writes idx[0..k) and val[0..k) and returns k.  Returns -1 if n < 0 or if
 * n exceeds the int32 index range ([VERL] risks section: positions are int32
 * on the wire and would wrap silently past 2^31 elements; this fails loudly).
 *
 * Pins: apply(old, diff(old,new)) == new; every returned index really differs;
 * strictly ascending; identical inputs give k == 0; equality with numpy's
 * view-compare-nonzero formulation; brute-force absorption sweep.
 */
int64_t oracle_diff(const uint16_t *old_bits, const uint16_t *new_bits, int64_t n,
                    int32_t *idx, uint16_t *val)
{
    int64_t i, k = 0;
    if (n < 0 || n > ORACLE_INT32_MAX)
        return -1;
    for (i = 0; i < n; ++i) {
        if (old_bits[i] != new_bits[i]) {
            idx[k] = (int32_t)i;
            val[k] = new_bits[i];
            ++k;
        }
    }
    return k;
}

/*
 * oracle_diff_many -- the batched form over a parameter list.
 *
 * [VERL] code-snippet section, `gather_v_batched_to_rank0`: the deltas of K
 * parameters are concatenated in list order together with a per-parameter
 * count vector; encode.py `DeltaParam` records each parameter's start/end in
 * the concatenated positions and values.
 *
 * Indices stay parameter-local.  nnz[p] is parameter p's change count and
 * offsets[p] the running sum (offsets has nparams+1 entries).  Writes at most
 * `capacity` entries into idx/val but always reports the true counts.
 * Returns 0, or -1 on a negative or over-long parameter.
 *
 * Pins: equals the per-parameter oracle_diff results appended in order.
 */
int oracle_diff_many(int32_t nparams, const uint16_t *const *olds,
                     const uint16_t *const *news, const int64_t *numels,
                     int32_t *idx, uint16_t *val, int64_t capacity,
                     int64_t *nnz, int64_t *offsets)
{
    int32_t p;
    int64_t i, k = 0;
    if (nparams < 0)
        return -1;
    for (p = 0; p < nparams; ++p)
        if (numels[p] < 0 || numels[p] > ORACLE_INT32_MAX)
            return -1;
    for (p = 0; p < nparams; ++p) {
        int64_t start = k;
        offsets[p] = start;
        for (i = 0; i < numels[p]; ++i) {
            if (olds[p][i] != news[p][i]) {
                if (k < capacity) {
                    idx[k] = (int32_t)i;
                    val[k] = news[p][i];
                }
                ++k;
            }
        }
        nnz[p] = k - start;
    }
    offsets[nparams] = k;
    return 0;
}

/*
 * oracle_shard_delta_many -- the sharded form: each parameter is one rank's
 * local shard of a larger parameter, and positions are made global.
 *
 * [VERL] code-snippet section, sparse_gather.py `shard_delta_indices`: the
 * local shard is compared bytewise exactly like a whole tensor, and every
 * local index is shifted by the shard's flat offset into the full parameter,
 * widened to int64.  spec.py `derive_placement`: under Shard(0) that flat
 * offset is the shard's first row times the product of the remaining
 * dimensions (computed by the caller and passed in flat_offsets).
 *
 * Same layout as oracle_diff_many (list order, per-parameter counts and
 * running offsets, at most `capacity` entries written, true counts always
 * reported), except that gidx is int64 and holds flat_offsets[p] + i.
 * Returns 0, or -1 on a negative or over-long shard or a negative offset.
 *
 * Pins: for row splits of a tensor as Shard(0) makes them (torch's own shard
 * size/offset routine), the shards' outputs concatenated in rank order equal
 * oracle_diff of the whole tensor, widened; an offset past 2^31 stays exact;
 * offset 0 reproduces oracle_diff_many.
 */
int oracle_shard_delta_many(int32_t nparams, const uint16_t *const *olds,
                            const uint16_t *const *news, const int64_t *numels,
                            const int64_t *flat_offsets, int64_t *gidx, uint16_t *val,
                            int64_t capacity, int64_t *nnz, int64_t *offsets)
{
    int32_t p;
    int64_t i, k = 0;
    if (nparams < 0)
        return -1;
    for (p = 0; p < nparams; ++p)
        if (numels[p] < 0 || numels[p] > ORACLE_INT32_MAX || flat_offsets[p] < 0)
            return -1;
    for (p = 0; p < nparams; ++p) {
        int64_t start = k;
        offsets[p] = start;
        for (i = 0; i < numels[p]; ++i) {
            if (olds[p][i] != news[p][i]) {
                if (k < capacity) {
                    gidx[k] = flat_offsets[p] + i;
                    val[k] = news[p][i];
                }
                ++k;
            }
        }
        nnz[p] = k - start;
    }
    offsets[nparams] = k;
    return 0;
}

/*
 * oracle_apply -- scatter the delta into the resident snapshot, in place.
 *
 * [TRL] section 4.3 (the vLLM-side extension): the receiver flattens its bf16
 * snapshot and assigns the values at the indices; the vLLM sparse-transfer
 * work mentioned there applies (indices, values) in place with index_copy_.
 * [VERL] implementation section, SGLang delta loader: in-place masked copy.
 *
 * Precondition checked first, before any write: indices are strictly
 * ascending and inside [0, n).  Returns 0, or -1 on a violation (snapshot
 * untouched) or on nnz < 0.
 *
 * Pins: apply(old, diff(old,new)) == new, untouched positions keep their bits,
 * replay over two steps, the reverse delta restores old.
 */
int oracle_apply(uint16_t *snap, int64_t n, const int32_t *idx, const uint16_t *val,
                 int64_t nnz)
{
    int64_t j;
    if (nnz < 0 || n < 0)
        return -1;
    for (j = 0; j < nnz; ++j) {
        if (idx[j] < 0 || (int64_t)idx[j] >= n)
            return -1;
        if (j > 0 && idx[j] <= idx[j - 1])
            return -1;
    }
    for (j = 0; j < nnz; ++j)
        snap[idx[j]] = val[j];
    return 0;
}

/*
 * oracle_xor_mask / oracle_xor_apply -- the XOR-mask mode.
 *
 * [XOR] first paragraph: the trainer takes a bitwise XOR of old and new
 * weights, giving a mask the size of the model in which a 1 bit marks a
 * flipped bit; the sampler XORs that mask into its old weights to obtain the
 * new ones, with no floating-point arithmetic.
 *
 * Pins: old ^ mask == new exactly; xor_apply is self-inverse; the nonzero
 * positions of the mask are exactly the diff indices.
 */
void oracle_xor_mask(const uint16_t *old_bits, const uint16_t *new_bits, uint16_t *mask,
                     int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        mask[i] = (uint16_t)(old_bits[i] ^ new_bits[i]);
}

void oracle_xor_apply(uint16_t *snap, const uint16_t *mask, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        snap[i] = (uint16_t)(snap[i] ^ mask[i]);
}

/*
 * oracle_bf16_rne -- round a double to the nearest bf16, ties to even.
 *
 * Written from the IEEE 754 binary-format definition: bf16 has 1 sign bit, an
 * 8-bit exponent with bias 127 and 7 stored significand bits, gradual
 * underflow below 2^-126 (spacing 2^-133), and results whose magnitude reaches
 * the largest finite value plus half its spacing round to infinity.  The
 * sign of a result that rounds to zero is the sign of the exact value.
 * [TRL] section 2 (why bf16 RL weights are almost always sparse): an update
 * smaller than half the spacing around the weight is absorbed by the cast.
 *
 * Used only by the absorption test and the synthetic-step cross-check.
 * NaN maps to the quiet NaN 0x7FC0 with the input's sign.
 *
 * Pins: agrees with torch's float32 -> bfloat16 cast on float32 inputs;
 * closed-form absorption predicate over every finite bf16 value.
 */
uint16_t oracle_bf16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    int e2, E;
    double q, r, m, frac;

    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;

    /* a = f * 2^e2 with f in [0.5, 1): the binade is [2^(e2-1), 2^e2). */
    (void)frexp(a, &e2);
    E = e2 - 1;
    if (E > 127)
        return (uint16_t)(sign | 0x7F80u);

    /* Spacing of representable values around a. */
    q = (E < -126) ? ldexp(1.0, -133) : ldexp(1.0, E - 7);

    /* Round a/q (an exact scaling) to an integer, ties to even. */
    r = a / q;
    m = floor(r);
    frac = r - m;
    if (frac > 0.5 || (frac == 0.5 && fmod(m, 2.0) != 0.0))
        m += 1.0;

    if (E < -126) {
        /* Subnormal grid: m counts units of 2^-133.  m == 128 is 2^-126,
         * the smallest normal, whose encoding is exponent 1 mantissa 0 --
         * numerically the same bit pattern as 128. */
        return (uint16_t)(sign | (uint16_t)m);
    }
    /* Normal grid: m in [128, 256]; 256 carries into the next binade. */
    if (m >= 256.0) {
        E += 1;
        m = 128.0;
    }
    if (E > 127)
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)((int)m - 128));
}

/* Element-wise form of oracle_bf16_rne over an array (same routine, looped). */
void oracle_bf16_rne_array(const double *x, uint16_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(x[i]);
}

/*
 * oracle_sparsity -- the fraction of elements left unchanged.
 *
 * [TRL] section 4.1 (delta metadata carries `sparsity`) and section 4.2 (the
 * sync log prints changed/total elements and the sparsity as a percentage).
 * sparsity = 1 - changed / total; 0 for an empty model.
 *
 * Pin: the worked log line in section 4.2 (golden fixture).
 */
double oracle_sparsity(int64_t changed, int64_t total)
{
    if (total <= 0)
        return 0.0;
    return 1.0 - (double)changed / (double)total;
}

/*
 * oracle_touched_lines -- how many distinct L-byte snapshot lines a delta
 * writes, for the apply cost model (each touched line is read and written).
 * `base_byte_offset` is the snapshot's byte address modulo L.  Counts the
 * distinct values of (base + 2*idx[j]) / L over a strictly ascending idx.
 *
 * Pin: brute force against a Python set on small inputs.
 */
int64_t oracle_touched_lines(const int32_t *idx, int64_t nnz, int64_t line_bytes,
                             int64_t base_byte_offset)
{
    int64_t j, g = 0, prev = -1;
    for (j = 0; j < nnz; ++j) {
        int64_t line = (base_byte_offset + 2 * (int64_t)idx[j]) / line_bytes;
        if (line != prev) {
            ++g;
            prev = line;
        }
    }
    return g;
}

/*
 * Wire encoding of a batched delta ([VERL] encode.py: `DeltaParam`,
 * `DeltaFlush`, `checksum`).
 *
 * oracle_wire_width -- bytes per position of a parameter: the pages give a
 * width of 2 or 4 bytes per parameter; the reading taken is the narrowest
 * that holds every parameter-local index, i.e. 2 when numel <= 65536.
 */
int oracle_wire_width(int64_t numel)
{
    return numel <= 65536 ? 2 : 4;
}

/*
 * oracle_wire_encode -- the positions byte block: parameter by parameter in
 * list order, each parameter-local index of the delta written little-endian
 * with that parameter's width.  pos_offsets (nparams+1 entries) receives
 * each parameter's start in the block (`pos_start`; the next entry is its
 * `pos_end`).  Returns the block's size in bytes, or -1 on bad arguments.
 *
 * Pins: the bytes equal numpy's per-segment astype('<u2' / '<u4') bytes;
 * oracle_wire_decode inverts it exactly.
 */
int64_t oracle_wire_encode(int32_t nparams, const int64_t *numels, const int32_t *idx,
                           const int64_t *offsets, uint8_t *positions, int64_t *pos_offsets)
{
    int32_t p;
    int64_t j, at = 0;
    if (nparams < 0)
        return -1;
    for (p = 0; p < nparams; ++p) {
        int w = oracle_wire_width(numels[p]);
        pos_offsets[p] = at;
        for (j = offsets[p]; j < offsets[p + 1]; ++j) {
            uint32_t v = (uint32_t)idx[j];
            int b;
            for (b = 0; b < w; ++b)
                positions[at + b] = (uint8_t)(v >> (8 * b));
            at += w;
        }
    }
    pos_offsets[nparams] = at;
    return at;
}

/*
 * oracle_wire_decode -- back from the byte block to int32 parameter-local
 * indices (the layout oracle_diff_many writes).  Returns 0.
 */
int oracle_wire_decode(int32_t nparams, const int64_t *numels, const uint8_t *positions,
                       const int64_t *pos_offsets, const int64_t *offsets, int32_t *idx)
{
    int32_t p;
    int64_t j;
    for (p = 0; p < nparams; ++p) {
        int w = oracle_wire_width(numels[p]);
        int64_t at = pos_offsets[p];
        for (j = offsets[p]; j < offsets[p + 1]; ++j) {
            uint32_t v = 0;
            int b;
            for (b = 0; b < w; ++b)
                v |= (uint32_t)positions[at + b] << (8 * b);
            idx[j] = (int32_t)v;
            at += w;
        }
    }
    return 0;
}

/*
 * oracle_hash_bytes / oracle_hash_bf16 -- the two halves of the flush
 * checksum ([VERL] encode.py `checksum`): torch.hash_tensor's XOR reduction
 * of the elements widened to 64 bits -- bytes zero-extended; bf16 values
 * widened to IEEE double (through float, as C converts) and taken as their
 * bit patterns.  The checksum itself is hash_bytes ^ (hash_bf16 << 1) as an
 * unbounded integer (the pages compute it on Python ints).
 *
 * Pins: equal to torch.hash_tensor on the same tensors, for every one of the
 * 65536 bf16 patterns and for random arrays.
 */
uint64_t oracle_hash_bytes(const uint8_t *bytes, int64_t n)
{
    int64_t i;
    uint64_t h = 0;
    for (i = 0; i < n; ++i)
        h ^= (uint64_t)bytes[i];
    return h;
}

uint64_t oracle_hash_bf16(const uint16_t *bits, int64_t n)
{
    int64_t i;
    uint64_t h = 0;
    for (i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)bits[i] << 16;
        float f;
        double d;
        uint64_t b;
        memcpy(&f, &u, sizeof f);
        d = (double)f;
        memcpy(&b, &d, sizeof b);
        h ^= b;
    }
    return h;
}

/*
 * Blocked positions: a 2-byte position for every parameter, whatever its size.
 *
 * [VERL] encode.py `DeltaParam.pos_width` sends positions at 2 or 4 bytes.
 * A parameter of more than 65536 elements cannot use 2 bytes as such; the
 * reading taken here (the pages do not give one) cuts its index range into
 * blocks of 65536 elements.  A position is stored as its offset inside its
 * block, 2 bytes little-endian; each block stores, 4 bytes little-endian, the
 * number of the parameter's entries that lie before it (the block's base in
 * the parameter's entry list; its base element is its number times 65536).
 * A flush's blocked positions are one byte block: first the block tables of
 * all parameters in list order (ceil(numel / 65536) words each), then the
 * 2-byte offsets of all entries in entry order.  Decoding entry j of
 * parameter p takes the last block b whose base is at most j - offsets[p]
 * and gives 65536 * b + offset.
 *
 * oracle_wire_blocked_size -- the block's size in bytes for `entries`
 * entries over the list: 4 bytes per 65536-element block plus 2 per entry.
 */
int64_t oracle_wire_blocked_size(int32_t nparams, const int64_t *numels, int64_t entries)
{
    int32_t p;
    int64_t blocks = 0;
    if (nparams < 0 || entries < 0)
        return -1;
    for (p = 0; p < nparams; ++p) {
        if (numels[p] < 0)
            return -1;
        blocks += (numels[p] + 65535) / 65536;
    }
    return 4 * blocks + 2 * entries;
}

/*
 * oracle_wire_encode_blocked -- writes the blocked positions of a
 * diff_many-layout delta (parameter-local idx, offsets[nparams+1]) to `out`
 * and returns their size, or -1 if an index is outside its parameter or
 * not strictly above its predecessor (the delta's own invariant, which the
 * block bases rely on).  A block's base is the count of the parameter's
 * entries below the block's first element, found by walking the entries
 * once in ascending order.
 *
 * Pins: a hand-written worked example (tests/golden/wire_blocked.txt); the
 * bases equal numpy's searchsorted of the block starts and the offsets its
 * '<u2' bytes of idx & 0xFFFF; oracle_wire_decode_blocked inverts it.
 */
int64_t oracle_wire_encode_blocked(int32_t nparams, const int64_t *numels, const int32_t *idx,
                                   const int64_t *offsets, uint8_t *out)
{
    int32_t p;
    int64_t j, total, table_bytes, t = 0;
    if (nparams < 0)
        return -1;
    total = offsets[nparams] - offsets[0];
    table_bytes = oracle_wire_blocked_size(nparams, numels, 0);
    if (total < 0 || table_bytes < 0)
        return -1;
    for (p = 0; p < nparams; ++p) {
        int64_t nb = (numels[p] + 65535) / 65536, b;
        int64_t begin = offsets[p], end = offsets[p + 1];
        for (j = begin; j < end; ++j) {
            if (idx[j] < 0 || idx[j] >= numels[p] || (j > begin && idx[j] <= idx[j - 1]))
                return -1;
        }
        j = begin;
        for (b = 0; b < nb; ++b) {
            uint32_t base;
            while (j < end && (int64_t)idx[j] < b * 65536)
                ++j;
            base = (uint32_t)(j - begin);
            out[4 * t + 0] = (uint8_t)(base);
            out[4 * t + 1] = (uint8_t)(base >> 8);
            out[4 * t + 2] = (uint8_t)(base >> 16);
            out[4 * t + 3] = (uint8_t)(base >> 24);
            ++t;
        }
    }
    for (j = offsets[0]; j < offsets[nparams]; ++j) {
        uint32_t off = (uint32_t)idx[j] & 0xFFFFu;
        out[table_bytes + 2 * (j - offsets[0]) + 0] = (uint8_t)off;
        out[table_bytes + 2 * (j - offsets[0]) + 1] = (uint8_t)(off >> 8);
    }
    return table_bytes + 2 * total;
}

/*
 * oracle_wire_decode_blocked -- the int32 parameter-local indices back from
 * `nbytes` bytes of blocked positions.  Returns 0, or -1 if the bytes are too
 * few for the list's tables and entries or a table is not a non-decreasing
 * run of bases from 0 within the parameter's entry count (the entries
 * decoded before the fault are written; the rest of idx is left alone).
 */
int oracle_wire_decode_blocked(int32_t nparams, const int64_t *numels, const uint8_t *in,
                               int64_t nbytes, const int64_t *offsets, int32_t *idx)
{
    int32_t p;
    int64_t t = 0, table_bytes, total;
    if (nparams < 0)
        return -1;
    total = offsets[nparams] - offsets[0];
    table_bytes = oracle_wire_blocked_size(nparams, numels, 0);
    if (total < 0 || table_bytes < 0 || nbytes < table_bytes + 2 * total)
        return -1;
    for (p = 0; p < nparams; ++p) {
        int64_t nb = (numels[p] + 65535) / 65536, b;
        int64_t count = offsets[p + 1] - offsets[p];
        for (b = 0; b < nb; ++b) {
            const uint8_t *w = in + 4 * (t + b);
            int64_t base = (int64_t)w[0] | ((int64_t)w[1] << 8) | ((int64_t)w[2] << 16) |
                           ((int64_t)w[3] << 24);
            int64_t next = count, k;
            if (b + 1 < nb) {
                const uint8_t *x = w + 4;
                next = (int64_t)x[0] | ((int64_t)x[1] << 8) | ((int64_t)x[2] << 16) |
                       ((int64_t)x[3] << 24);
            }
            if ((b == 0 && base != 0) || base > next || next > count)
                return -1;
            for (k = base; k < next; ++k) {
                int64_t j = offsets[p] + k;
                const uint8_t *h = in + table_bytes + 2 * (j - offsets[0]);
                idx[j] = (int32_t)(65536 * b + ((int64_t)h[0] | ((int64_t)h[1] << 8)));
            }
        }
        t += nb;
    }
    return 0;
}
