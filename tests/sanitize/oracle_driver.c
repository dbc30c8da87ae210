/* Drives every form of the CPU oracle on inputs held in buffers of exactly their length,
 * for a build under AddressSanitizer and UndefinedBehaviorSanitizer: any read past a
 * message's last byte, any leak and any undefined operation ends the run with an error.
 * The forms must also agree with each other (exit status 1 otherwise). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct b3o_hasher b3o_hasher;
void b3o_hash_recursive(const uint8_t *data, uint64_t len, const uint8_t *key32, uint8_t out32[32]);
void b3o_keyed_hash(const uint8_t *data, uint64_t len, const uint8_t key32[32], uint8_t out32[32]);
void b3o_hash(const uint8_t *data, uint64_t len, uint8_t out32[32]);
int b3o_hash_mt(const uint8_t *data, uint64_t len, const uint8_t *key32, uint8_t out32[32], int nthreads);
b3o_hasher *b3o_hasher_new(const uint8_t *key32);
void b3o_hasher_update(b3o_hasher *h, const uint8_t *data, uint64_t len);
void b3o_hasher_finalize(const b3o_hasher *h, uint8_t out32[32]);
void b3o_hasher_free(b3o_hasher *h);
void b3o_subtree_cv(const uint8_t *data, uint64_t len, uint64_t chunk_base, const uint8_t *key32, uint32_t out[8]);
void b3o_hash_xof_at(const uint8_t *data, uint64_t len, const uint8_t *key32, uint64_t offset, uint8_t *out,
                     uint64_t out_len);
int b3o_hash_batch(const uint8_t *base, const uint64_t *offsets, const uint64_t *lengths, uint64_t n,
                   const uint8_t *keys32, uint8_t *out, int nthreads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* xorshift64 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}

static uint8_t *random_buffer(uint64_t len) {
    uint8_t *p = (uint8_t *)malloc(len ? len : 1);
    for (uint64_t i = 0; i < len; ++i) p[i] = (uint8_t)next_u64();
    return p;
}

static int fail(const char *what, uint64_t len) {
    fprintf(stderr, "forms disagree: %s, length %llu\n", what, (unsigned long long)len);
    return 1;
}

int main(void) {
    static const uint64_t lengths[] = {0, 1, 63, 64, 65, 1023, 1024, 1025, 2048, 3 * 1024 + 1,
                                       13 * 1024 + 17, 64 * 1024 + 7, 300 * 1024 + 5};
    const size_t n_len = sizeof(lengths) / sizeof(lengths[0]);
    uint8_t key[32];
    for (int i = 0; i < 32; ++i) key[i] = (uint8_t)next_u64();
    for (size_t li = 0; li < n_len; ++li) {
        const uint64_t len = lengths[li];
        uint8_t *data = random_buffer(len);
        for (int keyed = 0; keyed < 2; ++keyed) {
            const uint8_t *k = keyed ? key : NULL;
            uint8_t a[32], b[32], c[32], d[32];
            b3o_hash_recursive(data, len, k, a);
            if (keyed) b3o_keyed_hash(data, len, key, b);
            else b3o_hash(data, len, b);
            if (b3o_hash_mt(data, len, k, c, 4) != 0) return fail("multi-threaded form failed", len);
            b3o_hasher *h = b3o_hasher_new(k);
            for (uint64_t at = 0; at < len;) { /* random update sizes, 1-byte ones included */
                uint64_t step = 1 + next_u64() % 1500;
                if (step > len - at) step = len - at;
                b3o_hasher_update(h, data + at, step);
                at += step;
            }
            b3o_hasher_finalize(h, d);
            b3o_hasher_free(h);
            if (memcmp(a, b, 32) || memcmp(a, c, 32) || memcmp(a, d, 32)) return fail("hash", len);
            /* extended output: a read from an offset equals the same bytes of a read from 0 */
            const uint64_t out_len = 200;
            uint8_t *whole = (uint8_t *)malloc(out_len + 100);
            uint8_t *part = (uint8_t *)malloc(out_len);
            b3o_hash_xof_at(data, len, k, 0, whole, out_len + 100);
            b3o_hash_xof_at(data, len, k, 100, part, out_len);
            if (memcmp(whole, a, 32) || memcmp(whole + 100, part, out_len)) return fail("xof", len);
            b3o_hash_xof_at(data, len, k, (1ull << 38) - 5, part, 17); /* across the 2^32-block boundary */
            free(whole);
            free(part);
            uint32_t cv[8];
            b3o_subtree_cv(data, len, 1ull << 33, k, cv);
        }
        free(data);
    }
    /* a batch in one buffer of exactly its size, the last message ending at its last byte */
    enum { N = 7 };
    const uint64_t blen[N] = {0, 1, 1024, 1025, 65, 4096 + 3, 2 * 1024 + 9};
    uint64_t boff[N], total = 0;
    for (int i = 0; i < N; ++i) {
        boff[i] = total;
        total += blen[i];
    }
    uint8_t *base = random_buffer(total);
    uint8_t *keys = random_buffer(32 * N);
    uint8_t *outs = (uint8_t *)malloc(32 * N);
    if (b3o_hash_batch(base, boff, blen, N, keys, outs, 3) != 0) return fail("batch failed", total);
    for (int i = 0; i < N; ++i) {
        uint8_t one[32];
        b3o_keyed_hash(base + boff[i], blen[i], keys + 32 * i, one);
        if (memcmp(one, outs + 32 * i, 32)) return fail("batch", blen[i]);
    }
    free(base);
    free(keys);
    free(outs);
    puts("oracle driver: all forms agree");
    return 0;
}
