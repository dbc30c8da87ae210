/*
 * blake3_oracle.c - plain, slow, scalar CPU BLAKE3 used as the parity oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg do. It
 * shares no code, header, table or helper with the HIP library.
 *
 * What it computes. The BLAKE3 hash (default or keyed mode, 32-byte output) of a byte
 * string. The page "BLAKE3 on GPU: 400x faster hashing" (qfminer.top, section
 * "BLAKE3") describes the method in prose: 1024-byte chunks, each compressed as
 * sequential 64-byte blocks by a 7-round add/xor/rotate compression function with a
 * message permutation between rounds; a 32-byte chaining value (CV) carried from block
 * to block, starting at the IV or, in keyed mode, at the key; a flag set, block length
 * and per-chunk counter as further inputs; then a binary tree of parent compressions
 * over the chunk CVs whose shape obeys "left subtree full" and "left subtree at least
 * as large as its right sibling". The page names the BLAKE3 specification for that
 * shape and gives no constants; the constants and the exact state layout below are the
 * published BLAKE3 specification's (O'Connor, Aumasson, Neves, Wilcox-O'Hearn, 2020),
 * restated here in this file's own code.
 *
 * Pins (see tests/test_oracle_pins.py): IV from its closed form; G, rotations, IV and
 * the column/diagonal round layout via a BLAKE2s built on b3o_round() that must equal
 * Python's hashlib.blake2s; the two tree-shape rules and the page's 13 = 8+4+1 example
 * ("Merkle tree reduction"); recursive form == stack-merge form == incremental form ==
 * multi-threaded form. The message permutation, flag values and the counter/length/flag
 * words of the state are fixed by the keyed-hash cross-check against an independent
 * BLAKE3 (the Xet client library's). The extended output (tests/test_oracle_xof.py) is
 * tied to the digest, and each of its 64-byte blocks must invert, through the test's own
 * inverse rounds, to the root node's input state with its block counter. Default mode's
 * flag value 0 rests on the specification text alone: "parity unpinned".
 *
 * The form here follows the definitions literally: no SIMD, no blocking, no fusion.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define B3O_CHUNK_LEN 1024u
#define B3O_BLOCK_LEN 64u
#define B3O_KEY_LEN 32u
#define B3O_OUT_LEN 32u

/* Domain-separation flags (specification, "Compression function", flag table). The
 * page names CHUNK_START, CHUNK_END, KEYED_HASH, PARENT and ROOT ("Compression
 * function", "Merkle tree reduction", "Kernels 2 and 3") without values. */
enum {
    B3O_CHUNK_START = 1u << 0,
    B3O_CHUNK_END = 1u << 1,
    B3O_PARENT = 1u << 2,
    B3O_ROOT = 1u << 3,
    B3O_KEYED_HASH = 1u << 4,
};

/* IV: first 32 bits of the fractional parts of the square roots of the first eight
 * primes (specification, "Compression function"; the page only says "some IV"). */
static const uint32_t B3O_IV[8] = {
    0x6A09E667u, 0xBB67AE85u, 0x3C6EF372u, 0xA54FF53Au,
    0x510E527Fu, 0x9B05688Cu, 0x1F83D9ABu, 0x5BE0CD19u,
};

/* Message word permutation applied between rounds (specification, "Compression
 * function"): after permuting, new word i is old word B3O_PERM[i]. */
static const unsigned B3O_PERM[16] = {2, 6, 3, 10, 7, 0, 4, 13, 1, 11, 12, 5, 9, 14, 15, 8};

static uint32_t rotr32(uint32_t x, unsigned k) { return (x >> k) | (x << (32u - k)); }

static uint32_t load_le32(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static void store_le32(uint8_t *p, uint32_t w) {
    p[0] = (uint8_t)w;
    p[1] = (uint8_t)(w >> 8);
    p[2] = (uint8_t)(w >> 16);
    p[3] = (uint8_t)(w >> 24);
}

/* The quarter-round G on state words a,b,c,d with message words x,y. */
static void g(uint32_t v[16], int a, int b, int c, int d, uint32_t x, uint32_t y) {
    v[a] = v[a] + v[b] + x;
    v[d] = rotr32(v[d] ^ v[a], 16);
    v[c] = v[c] + v[d];
    v[b] = rotr32(v[b] ^ v[c], 12);
    v[a] = v[a] + v[b] + y;
    v[d] = rotr32(v[d] ^ v[a], 8);
    v[c] = v[c] + v[d];
    v[b] = rotr32(v[b] ^ v[c], 7);
}

/* One round: G on the four columns, then on the four diagonals, consuming the message
 * words in order m[0..15]. Exported so the tests can build BLAKE2s on it. */
void b3o_round(uint32_t v[16], const uint32_t m[16]) {
    g(v, 0, 4, 8, 12, m[0], m[1]);
    g(v, 1, 5, 9, 13, m[2], m[3]);
    g(v, 2, 6, 10, 14, m[4], m[5]);
    g(v, 3, 7, 11, 15, m[6], m[7]);
    g(v, 0, 5, 10, 15, m[8], m[9]);
    g(v, 1, 6, 11, 12, m[10], m[11]);
    g(v, 2, 7, 8, 13, m[12], m[13]);
    g(v, 3, 4, 9, 14, m[14], m[15]);
}

void b3o_iv(uint32_t out[8]) { memcpy(out, B3O_IV, sizeof(B3O_IV)); }

/* The compression function: 16-word state from the CV, the first four IV words, the
 * 64-bit counter (low word, high word), the block length and the flags; seven rounds
 * with the message permuted between consecutive rounds; output word i is
 * v[i] ^ v[i+8] and, for the extended output, word i+8 is v[i+8] ^ cv[i]. */
void b3o_compress(const uint32_t cv[8], const uint32_t block_words[16], uint64_t counter,
                  uint32_t block_len, uint32_t flags, uint32_t out[16]) {
    uint32_t v[16], m[16], tmp[16];
    for (int i = 0; i < 8; i++) v[i] = cv[i];
    for (int i = 0; i < 4; i++) v[8 + i] = B3O_IV[i];
    v[12] = (uint32_t)counter;
    v[13] = (uint32_t)(counter >> 32);
    v[14] = block_len;
    v[15] = flags;
    memcpy(m, block_words, sizeof(m));
    for (int r = 0; r < 7; r++) {
        b3o_round(v, m);
        if (r < 6) {
            for (int i = 0; i < 16; i++) tmp[i] = m[B3O_PERM[i]];
            memcpy(m, tmp, sizeof(m));
        }
    }
    for (int i = 0; i < 8; i++) {
        out[i] = v[i] ^ v[i + 8];
        out[i + 8] = v[i + 8] ^ cv[i];
    }
}

/* Key words and mode flag for a hash: keyed mode starts every chunk and parent at the
 * key (read as eight little-endian words) and sets KEYED_HASH on every compression;
 * default mode uses the IV and no mode flag (page, "BLAKE3"; specification, "Modes"). */
static void mode_setup(const uint8_t *key32, uint32_t key_words[8], uint32_t *mode) {
    if (key32) {
        for (int i = 0; i < 8; i++) key_words[i] = load_le32(key32 + 4 * i);
        *mode = B3O_KEYED_HASH;
    } else {
        memcpy(key_words, B3O_IV, sizeof(B3O_IV));
        *mode = 0;
    }
}

static void words_from_block(const uint8_t *bytes, size_t n, uint32_t w[16]) {
    uint8_t block[B3O_BLOCK_LEN];
    memset(block, 0, sizeof(block));
    if (n) memcpy(block, bytes, n);
    for (int i = 0; i < 16; i++) w[i] = load_le32(block + 4 * i);
}

/* Chunk chaining (page, "BLAKE3" and "Compression function"): the chunk's bytes are cut
 * into max(1, ceil(len/64)) blocks; the CV starts at the key words; every block uses
 * the chunk index as counter; the first block carries CHUNK_START, the last carries
 * CHUNK_END (and ROOT when this chunk is the whole input); every block but the last
 * has length 64, the last has the remaining byte count, zero-padded. An empty chunk
 * (only the empty input) is one zero block of length 0. */
void b3o_chunk_cv(const uint32_t key_words[8], uint32_t mode, const uint8_t *chunk, size_t len,
                  uint64_t chunk_index, int is_root, uint32_t out[8]) {
    size_t nblocks = len == 0 ? 1 : (len + B3O_BLOCK_LEN - 1) / B3O_BLOCK_LEN;
    uint32_t cv[8], m[16], o[16];
    memcpy(cv, key_words, sizeof(cv));
    for (size_t b = 0; b < nblocks; b++) {
        size_t off = b * B3O_BLOCK_LEN;
        size_t blen = (b + 1 == nblocks) ? len - off : B3O_BLOCK_LEN;
        uint32_t flags = mode;
        if (b == 0) flags |= B3O_CHUNK_START;
        if (b + 1 == nblocks) {
            flags |= B3O_CHUNK_END;
            if (is_root) flags |= B3O_ROOT;
        }
        words_from_block(chunk + off, blen, m);
        b3o_compress(cv, m, chunk_index, (uint32_t)blen, flags, o);
        memcpy(cv, o, sizeof(cv));
    }
    memcpy(out, cv, sizeof(cv));
}

/* Parent node (page, "Merkle tree reduction"): the two child CVs concatenated as one
 * 64-byte block, compressed from the key words with counter 0, block length 64 and
 * flags mode|PARENT (|ROOT for the final compression). */
void b3o_parent_cv(const uint32_t key_words[8], uint32_t mode, const uint32_t left[8],
                   const uint32_t right[8], int is_root, uint32_t out[8]) {
    uint32_t m[16], o[16];
    memcpy(m, left, 8 * sizeof(uint32_t));
    memcpy(m + 8, right, 8 * sizeof(uint32_t));
    b3o_compress(key_words, m, 0, B3O_BLOCK_LEN, mode | B3O_PARENT | (is_root ? B3O_ROOT : 0), o);
    memcpy(out, o, 8 * sizeof(uint32_t));
}

/* Number of chunks in the left subtree of a node over n > 1 chunks: the largest power
 * of two strictly below n. It is the only split the two shape rules of the page
 * ("BLAKE3": left subtree complete with a power-of-two chunk count; left subtree at
 * least as large as the right one) allow, since exactly one power of two lies in
 * [n/2, n). */
uint64_t b3o_left_subtree_chunks(uint64_t n) {
    uint64_t k = 1;
    while (k * 2 < n) k *= 2;
    return k;
}

static uint64_t num_chunks(uint64_t len) {
    return len == 0 ? 1 : (len + B3O_CHUNK_LEN - 1) / B3O_CHUNK_LEN;
}

/* CV of the subtree over chunks [first, first+n) of the input, whose chunk 0 has counter
 * `base`; ROOT only at the top of the whole tree. This is the recursive definition of
 * the tree. */
static void subtree_cv(const uint32_t kw[8], uint32_t mode, const uint8_t *data, uint64_t len, uint64_t base,
                       uint64_t first, uint64_t n, int is_root, uint32_t out[8]) {
    if (n == 1) {
        uint64_t off = first * B3O_CHUNK_LEN;
        uint64_t clen = len - off < B3O_CHUNK_LEN ? len - off : B3O_CHUNK_LEN;
        b3o_chunk_cv(kw, mode, data + off, (size_t)clen, base + first, is_root, out);
        return;
    }
    uint64_t k = b3o_left_subtree_chunks(n);
    uint32_t l[8], r[8];
    subtree_cv(kw, mode, data, len, base, first, k, 0, l);
    subtree_cv(kw, mode, data, len, base, first + k, n - k, 0, r);
    b3o_parent_cv(kw, mode, l, r, is_root, out);
}

static void words_to_bytes(const uint32_t w[8], uint8_t out32[32]) {
    for (int i = 0; i < 8; i++) store_le32(out32 + 4 * i, w[i]);
}

/* Recursive (top-down) form of the whole hash. key32 == NULL selects default mode. */
void b3o_hash_recursive(const uint8_t *data, uint64_t len, const uint8_t *key32, uint8_t out32[32]) {
    uint32_t kw[8], mode, root[8];
    mode_setup(key32, kw, &mode);
    subtree_cv(kw, mode, data, len, 0, 0, num_chunks(len), 1, root);
    words_to_bytes(root, out32);
}

/* CV (8 words, no ROOT) of the subtree formed by all chunks of data[0 .. len), where
 * chunk 0 has counter chunk_base: a node of the tree of a larger input when data is an
 * aligned part of it. key32 == NULL selects default mode. */
void b3o_subtree_cv(const uint8_t *data, uint64_t len, uint64_t chunk_base, const uint8_t *key32,
                    uint32_t out[8]) {
    uint32_t kw[8], mode;
    mode_setup(key32, kw, &mode);
    subtree_cv(kw, mode, data, len, chunk_base, 0, num_chunks(len), 0, out);
}

/* ---- Extended output (XOF) ---------------------------------------------------------
 * The root node is the tree's final compression: for a one-chunk input, the chunk's
 * last block, with the CV chained through the earlier blocks; otherwise the parent of
 * the two top subtrees (left: the largest power of two of chunks below n). Output block
 * t (64 bytes) is that compression run again with counter t and ROOT, all sixteen output
 * words (specification, "Extendable output"); its first 32 bytes for t = 0 are the hash.
 * b3o_hash_xof_at writes stream bytes [offset, offset + out_len), so any part of the stream
 * can be read without the blocks before it. The page leaves extendable output out ("Future
 * work"). key32 == NULL: default mode. */
void b3o_hash_xof_at(const uint8_t *data, uint64_t len, const uint8_t *key32, uint64_t offset, uint8_t *out,
                     uint64_t out_len) {
    uint32_t kw[8], mode, cv[8], m[16], o[16], blen, flags;
    mode_setup(key32, kw, &mode);
    uint64_t n = num_chunks(len);
    if (n == 1) {
        size_t nblocks = len == 0 ? 1 : (size_t)((len + B3O_BLOCK_LEN - 1) / B3O_BLOCK_LEN);
        memcpy(cv, kw, sizeof(cv));
        for (size_t b = 0; b + 1 < nblocks; b++) {
            words_from_block(data + b * B3O_BLOCK_LEN, B3O_BLOCK_LEN, m);
            b3o_compress(cv, m, 0, B3O_BLOCK_LEN, mode | (b == 0 ? B3O_CHUNK_START : 0), o);
            memcpy(cv, o, sizeof(cv));
        }
        size_t off = (nblocks - 1) * B3O_BLOCK_LEN;
        blen = (uint32_t)(len - off);
        words_from_block(data + off, blen, m);
        flags = mode | B3O_CHUNK_END | (nblocks == 1 ? B3O_CHUNK_START : 0);
    } else {
        uint64_t k = b3o_left_subtree_chunks(n);
        subtree_cv(kw, mode, data, len, 0, 0, k, 0, m);
        subtree_cv(kw, mode, data, len, 0, k, n - k, 0, m + 8);
        memcpy(cv, kw, sizeof(cv));
        blen = B3O_BLOCK_LEN;
        flags = mode | B3O_PARENT;
    }
    /* stream byte s = offset + j lies in block s / 64 at position s % 64 */
    for (uint64_t j = 0; j < out_len;) {
        uint64_t s = offset + j, t = s / B3O_BLOCK_LEN;
        uint8_t block[B3O_BLOCK_LEN];
        b3o_compress(cv, m, t, blen, flags | B3O_ROOT, o);
        for (int i = 0; i < 16; i++) store_le32(block + 4 * i, o[i]);
        uint64_t at = s % B3O_BLOCK_LEN, take = B3O_BLOCK_LEN - at;
        if (take > out_len - j) take = out_len - j;
        memcpy(out + j, block + at, (size_t)take);
        j += take;
    }
}

/* The first out_len bytes of the stream. */
void b3o_hash_xof(const uint8_t *data, uint64_t len, const uint8_t *key32, uint8_t *out, uint64_t out_len) {
    b3o_hash_xof_at(data, len, key32, 0, out, out_len);
}

/* ---- Incremental (stack-merge) form --------------------------------------------- */

typedef struct {
    uint32_t key_words[8];
    uint32_t mode;
    uint32_t stack[64][8]; /* subtree CVs, at most one per level: 2^64 chunks max */
    int depth;
    uint64_t closed_chunks;                /* chunks already folded into the stack */
    uint8_t open_chunk[B3O_CHUNK_LEN];     /* bytes of the chunk still open */
    size_t open_len;
} b3o_hasher;

b3o_hasher *b3o_hasher_new(const uint8_t *key32) {
    b3o_hasher *h = (b3o_hasher *)calloc(1, sizeof(b3o_hasher));
    if (h) mode_setup(key32, h->key_words, &h->mode);
    return h;
}

void b3o_hasher_free(b3o_hasher *h) { free(h); }

/* Close the open (full) chunk: its CV enters the stack, and while the number of closed
 * chunks is even the top two subtrees are equal-sized siblings and merge. */
static void close_open_chunk(b3o_hasher *h) {
    uint32_t cv[8];
    b3o_chunk_cv(h->key_words, h->mode, h->open_chunk, h->open_len, h->closed_chunks, 0, cv);
    h->closed_chunks++;
    uint64_t c = h->closed_chunks;
    while ((c & 1) == 0) {
        h->depth--;
        b3o_parent_cv(h->key_words, h->mode, h->stack[h->depth], cv, 0, cv);
        c >>= 1;
    }
    memcpy(h->stack[h->depth], cv, sizeof(cv));
    h->depth++;
    h->open_len = 0;
}

/* A full chunk is closed only when more input arrives, because the last chunk of the
 * input must stay open to take ROOT when it is the only chunk. */
void b3o_hasher_update(b3o_hasher *h, const uint8_t *data, uint64_t len) {
    while (len > 0) {
        if (h->open_len == B3O_CHUNK_LEN) close_open_chunk(h);
        size_t take = B3O_CHUNK_LEN - h->open_len;
        if (take > len) take = (size_t)len;
        memcpy(h->open_chunk + h->open_len, data, take);
        h->open_len += take;
        data += take;
        len -= take;
    }
}

/* Finish: the open chunk's CV is merged with the stack entries from the top down; the
 * last merge (or, with an empty stack, the open chunk itself) carries ROOT. The hasher
 * is left unchanged, so finalize may be called again after more updates. */
void b3o_hasher_finalize(const b3o_hasher *h, uint8_t out32[32]) {
    uint32_t out[8];
    b3o_chunk_cv(h->key_words, h->mode, h->open_chunk, h->open_len, h->closed_chunks, h->depth == 0,
                 out);
    for (int i = h->depth - 1; i >= 0; i--)
        b3o_parent_cv(h->key_words, h->mode, h->stack[i], out, i == 0, out);
    words_to_bytes(out, out32);
}

void b3o_hash(const uint8_t *data, uint64_t len, uint8_t out32[32]) {
    b3o_hasher h;
    memset(&h, 0, sizeof(h));
    mode_setup(NULL, h.key_words, &h.mode);
    b3o_hasher_update(&h, data, len);
    b3o_hasher_finalize(&h, out32);
}

void b3o_keyed_hash(const uint8_t *data, uint64_t len, const uint8_t key32[32], uint8_t out32[32]) {
    b3o_hasher h;
    memset(&h, 0, sizeof(h));
    mode_setup(key32, h.key_words, &h.mode);
    b3o_hasher_update(&h, data, len);
    b3o_hasher_finalize(&h, out32);
}

/* ---- Multi-threaded form (timing baseline) ---------------------------------------
 * The chunk range is cut into aligned groups of 2^s chunks (only the last may be
 * shorter). Because every split of the tree over n > 2^s chunks falls on a multiple of
 * 2^s, the tree over the input is the same shape rule applied to the group CVs; each
 * group's CV is computed by the recursive form without ROOT, then the group CVs are
 * combined by the same recursion with ROOT at the top. */

typedef struct {
    const uint32_t *kw;
    uint32_t mode;
    const uint8_t *data;
    uint64_t len, n_chunks, group_chunks, n_groups;
    uint32_t (*group_cv)[8];
    uint64_t next_group;
    pthread_mutex_t lock;
} mt_job;

static void *mt_worker(void *arg) {
    mt_job *job = (mt_job *)arg;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        uint64_t gidx = job->next_group++;
        pthread_mutex_unlock(&job->lock);
        if (gidx >= job->n_groups) break;
        uint64_t first = gidx * job->group_chunks;
        uint64_t n = job->n_chunks - first < job->group_chunks ? job->n_chunks - first : job->group_chunks;
        subtree_cv(job->kw, job->mode, job->data, job->len, 0, first, n, 0, job->group_cv[gidx]);
    }
    return NULL;
}

static void reduce_cvs(const uint32_t kw[8], uint32_t mode, uint32_t (*cvs)[8], uint64_t first, uint64_t n,
                       int is_root, uint32_t out[8]) {
    if (n == 1) {
        memcpy(out, cvs[first], 8 * sizeof(uint32_t));
        return;
    }
    uint64_t k = b3o_left_subtree_chunks(n);
    uint32_t l[8], r[8];
    reduce_cvs(kw, mode, cvs, first, k, 0, l);
    reduce_cvs(kw, mode, cvs, first + k, n - k, 0, r);
    b3o_parent_cv(kw, mode, l, r, is_root, out);
}

/* Returns 0 on success, -1 on allocation or thread failure. */
int b3o_hash_mt(const uint8_t *data, uint64_t len, const uint8_t *key32, uint8_t out32[32], int nthreads) {
    uint32_t kw[8], mode;
    mode_setup(key32, kw, &mode);
    uint64_t n = num_chunks(len);
    if (nthreads < 1) nthreads = 1;
    uint64_t group = 1;
    while (group * 2 <= n && (n + group * 2 - 1) / (group * 2) >= (uint64_t)(4 * nthreads)) group *= 2;
    uint64_t n_groups = (n + group - 1) / group;
    if (n_groups == 1 || nthreads == 1) {
        b3o_hash_recursive(data, len, key32, out32);
        return 0;
    }
    mt_job job;
    job.kw = kw;
    job.mode = mode;
    job.data = data;
    job.len = len;
    job.n_chunks = n;
    job.group_chunks = group;
    job.n_groups = n_groups;
    job.next_group = 0;
    job.group_cv = (uint32_t(*)[8])malloc(n_groups * sizeof(uint32_t[8]));
    if (!job.group_cv) return -1;
    pthread_mutex_init(&job.lock, NULL);
    pthread_t *tids = (pthread_t *)malloc((size_t)nthreads * sizeof(pthread_t));
    int started = 0, rc = 0;
    if (!tids) rc = -1;
    for (int t = 0; rc == 0 && t < nthreads; t++) {
        if (pthread_create(&tids[t], NULL, mt_worker, &job) != 0) rc = -1;
        else started++;
    }
    if (started == 0) mt_worker(&job);
    for (int t = 0; t < started; t++) pthread_join(tids[t], NULL);
    if (started > 0 && rc != 0) mt_worker(&job); /* finish any groups left over */
    uint32_t root[8];
    reduce_cvs(kw, mode, job.group_cv, 0, n_groups, 1, root);
    words_to_bytes(root, out32);
    pthread_mutex_destroy(&job.lock);
    free(tids);
    free(job.group_cv);
    return 0;
}

/* ---- Batch: many independent messages ---------------------------------------------
 * Each message is hashed on its own, with its own key (keys32 == NULL: default mode for
 * all), its own counter space starting at chunk 0 and its own ROOT. Messages are
 * shared among threads one at a time. */

typedef struct {
    const uint8_t *base;
    const uint64_t *offsets, *lengths;
    const uint8_t *keys32;
    uint8_t *out;
    uint64_t n, next;
    pthread_mutex_t lock;
} batch_job;

static void *batch_worker(void *arg) {
    batch_job *job = (batch_job *)arg;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        uint64_t i = job->next++;
        pthread_mutex_unlock(&job->lock);
        if (i >= job->n) break;
        b3o_hash_recursive(job->base + job->offsets[i], job->lengths[i],
                           job->keys32 ? job->keys32 + 32 * i : NULL, job->out + 32 * i);
    }
    return NULL;
}

int b3o_hash_batch(const uint8_t *base, const uint64_t *offsets, const uint64_t *lengths, uint64_t n,
                   const uint8_t *keys32, uint8_t *out, int nthreads) {
    batch_job job;
    job.base = base;
    job.offsets = offsets;
    job.lengths = lengths;
    job.keys32 = keys32;
    job.out = out;
    job.n = n;
    job.next = 0;
    pthread_mutex_init(&job.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t *tids = (pthread_t *)malloc((size_t)nthreads * sizeof(pthread_t));
    int started = 0;
    for (int t = 0; tids && t < nthreads; t++)
        if (pthread_create(&tids[t], NULL, batch_worker, &job) == 0) started++;
    batch_worker(&job);
    for (int t = 0; t < started; t++) pthread_join(tids[t], NULL);
    free(tids);
    pthread_mutex_destroy(&job.lock);
    return 0;
}
