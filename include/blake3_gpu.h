/*
 * blake3_gpu.h - C ABI of the MI355X (gfx950) BLAKE3 Merkle-tree hashing library.
 *
 * The library computes BLAKE3 digests (default or keyed mode, 32-byte output) of byte
 * buffers that already sit in GPU memory, with every step on the GPU and no host I/O of
 * the data. The operation is the one the page "BLAKE3 on GPU: 400x faster hashing"
 * (qfminer.top) describes: sections "BLAKE3" (1 KiB chunks of chained 64-byte block
 * compressions, keyed mode starting from the key, a binary tree of parent compressions
 * whose left subtree is complete and at least as large as the right one) and "Our
 * implementation" / "Kernels 2 and 3" (chunk compression fused with a partial tree
 * reduction, then level reductions ending in the ROOT-flagged final compression). The
 * requirements it meets are the introduction's: one GPU computation of a secure hash of
 * a single large device-resident input, using the whole GPU, without host I/O.
 *
 * Conventions for every entry point:
 *  - Pointers named dev_* are device pointers (HIP device memory, e.g. a torch tensor's
 *    data_ptr()); host_* and key are host pointers. The caller owns all of them; the
 *    library never frees or retains them after the call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). All work is
 *    enqueued on it; no entry point synchronises the host with the device. A digest is
 *    in dev_out once the stream reaches that point; read it after a stream sync. The
 *    stream and the dev_* buffers belong to the current device (hipSetDevice): scratch is
 *    taken on the current device.
 *  - Scratch (chaining values of intermediate tree levels, the batch task table) is
 *    library-owned device memory. Up to 64 MiB per call comes from a few slots per device
 *    that the library allocates on first use, grows when needed and keeps for the life of
 *    the process (memory a slot outgrows is kept too, never freed: freeing device or
 *    pinned memory would wait for every stream of the device): a call makes `stream` wait
 *    (on the device, not the host) until the slot's previous call has finished with it,
 *    and records its own completion for the next. Larger requests, calls that find every slot in use by other host threads, and
 *    calls on a stream under graph capture allocate and free their scratch in stream order
 *    on `stream` from a memory pool the library keeps per device. Calls on different
 *    streams and host threads may overlap; entry points are thread-safe.
 *  - Graph capture: on a stream being captured (hipStreamBeginCapture) an entry point
 *    records its kernels and its scratch's stream-ordered allocation and release; a
 *    replay hashes the input buffers' contents at replay time. Host key words are
 *    captured by value. The exception is a batch planned into a task table (one that is
 *    not uniform, below): its table is read from host memory that later calls reuse, so
 *    under capture it returns B3G_EINVAL and enqueues nothing.
 *  - Errors are returned as negative b3g_status values. Arguments are checked before any
 *    HIP call, so an argument error (EINVAL, EALIGN, ETOOBIG) enqueues nothing. ENOMEM and
 *    EHIP can come after part of the work was enqueued; the output is then unspecified.
 *    Faults of the device work itself (e.g. a dev_in that is not device memory) surface at
 *    the caller's next synchronisation.
 *  - Digests are the 8 output words of the final compression as little-endian bytes.
 */
#ifndef BLAKE3_GPU_H
#define BLAKE3_GPU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    B3G_OK = 0,
    B3G_EINVAL = -1,  /* a required pointer is NULL, or a batch offset + length overflows */
    B3G_EALIGN = -2,  /* dev_in, dev_base + offset or dev_keys is not 16-byte aligned */
    B3G_ENOMEM = -3,  /* scratch allocation failed */
    B3G_EHIP = -4,    /* a HIP runtime call or a kernel launch failed (incl. no device) */
    B3G_ETOOBIG = -5, /* the request exceeds what the planner represents (see below) */
    B3G_ESCRATCH = -6, /* blake3_gpu_keyed_hash_noalloc: the input needs more scratch than
                          its fixed array holds */
} b3g_status;

#define BLAKE3_GPU_KEY_WORDS 8
#define BLAKE3_GPU_OUT_LEN 32
/* Bytes of the fixed device array per GPU that blake3_gpu_keyed_hash_noalloc uses. */
#define BLAKE3_GPU_NOALLOC_SCRATCH_BYTES (1u << 20)

/*
 * Default-mode BLAKE3 of dev_in[0 .. len) (page, section "BLAKE3": without a key every
 * chunk and parent compression starts from the IV, and no mode flag is set).
 *   dev_in     device pointer, 16-byte aligned; may be NULL only when len == 0.
 *   len        byte count, 0 .. 2^42 (4 TiB; ETOOBIG above, so chunk indices fit 32 bits).
 *   dev_out32  device pointer to 32 writable bytes; receives the digest.
 * Errors: EINVAL (dev_out32 NULL, or dev_in NULL with len > 0), EALIGN, ETOOBIG, ENOMEM,
 * EHIP. The empty input is valid and yields the digest of one zero block of length 0.
 */
int blake3_gpu_hash(const void *dev_in, uint64_t len, void *dev_out32, void *stream);

/*
 * Keyed-mode BLAKE3 of dev_in[0 .. len) (page, section "BLAKE3": the key replaces the
 * IV as the starting chaining value of every chunk and parent; KEYED_HASH is set on
 * every compression).
 *   key        host pointer to 8 uint32 words: the 32-byte key read as little-endian
 *              words (byte 4*i is the low byte of key[i]). Copied by value into the
 *              kernel arguments; the buffer may be reused as soon as the call returns.
 * Other arguments and errors as blake3_gpu_hash; EINVAL also when key is NULL.
 */
int blake3_gpu_keyed_hash(const void *dev_in, uint64_t len, const uint32_t key[8], void *dev_out32,
                          void *stream);

/*
 * For callers that cannot allocate memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): blake3_gpu_keyed_hash (key != NULL) or blake3_gpu_hash
 * (key == NULL, default mode) with the same kernels and the same digests, that allocates
 * nothing. It calls no hipMalloc, hipFree, memory pool, event or pinned-buffer routine:
 * the chaining values between its launches live in a fixed array of
 * BLAKE3_GPU_NOALLOC_SCRATCH_BYTES (1 MiB) of device memory that the library holds on each
 * GPU it runs on until the process ends, instead of the scratch slots and pool of the other
 * entry points. The first call on a device looks up that device's address of the array
 * (hipGetSymbolAddress).
 *   Limit: the level CVs of the input must fit the array. In the default configuration
 *   that is at most 32,640 leaf workgroups of 1024 chunks: len <= 34,225,520,640 bytes
 *   (31.875 GiB). A larger input returns B3G_ESCRATCH before any HIP call.
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the last call's
 *   contents (no call depends on them: it writes every word it reads, and clears what must
 *   start at zero). Calls ordered on one stream are safe; calls that overlap on one GPU
 *   (unordered streams, host threads, or concurrently replayed graphs) race and may return
 *   wrong digests.
 * Arguments as blake3_gpu_keyed_hash, except that key may be NULL. Errors: EINVAL, EALIGN,
 * ETOOBIG, ESCRATCH, EHIP (never ENOMEM).
 */
int blake3_gpu_keyed_hash_noalloc(const void *dev_in, uint64_t len, const uint32_t key[8], void *dev_out32,
                                  void *stream);

/*
 * Many independent messages in one call (page, introduction: hashing many messages at once
 * is the common way to use a GPU; here each message gets its own tree): message i is
 * dev_base[host_offsets[i] .. host_offsets[i] + host_lengths[i]), hashed with its own key
 * and its own tree (counters restart at 0, each message gets its own ROOT).
 *   dev_base      device pointer, 16-byte aligned; may be NULL only if every length is 0.
 *   host_offsets  host array of n byte offsets, each a multiple of 16. Messages may be
 *                 in any order and may overlap (they are only read).
 *   host_lengths  host array of n byte counts (each 0 .. 2^42).
 *   dev_keys      device array of n*8 uint32 key words (message i's key at 8*i), 16-byte
 *                 aligned, or NULL for default (unkeyed) mode for every message.
 *   dev_out       device pointer to n*32 writable bytes; digest i at byte 32*i.
 *   n             message count (0 enqueues nothing and returns B3G_OK); at most 2^32-1
 *                 unless the batch is uniform (below).
 * The host arrays are read during the call only. A uniform batch (every length equal, and
 * offsets evenly spaced: offset i = offset 0 + i*d for one d, a multiple of 16, possibly
 * 0) needs no table: its launch geometry follows from (offset 0, d, length, n). Any other
 * batch is planned on the host into a task table that is copied to device scratch in
 * stream order before the call returns. Both give the same digests.
 * Errors: EINVAL (NULL arrays with n > 0, NULL dev_out, NULL dev_base with a non-empty
 * message, offset + length overflowing 64 bits), EALIGN (misaligned dev_base, offset or
 * dev_keys), ETOOBIG (a length above 2^42, or a planned pass of more workgroups than one
 * launch holds: 2^24 - 1 of 256 lanes, reached only by a table-planned batch of about
 * 16 TiB of message bytes, overlapping messages counted each time), ENOMEM, EHIP.
 */
int blake3_gpu_keyed_hash_batch(const void *dev_base, const uint64_t *host_offsets,
                                const uint64_t *host_lengths, const uint32_t *dev_keys, void *dev_out,
                                uint64_t n, void *stream);

/*
 * Chaining value of a subtree: the BLAKE3 tree over all chunks of dev_in[0 .. len) with
 * chunk counters starting at chunk_base, reduced to one 8-word CV with no ROOT flag
 * (page "BLAKE3 on GPU: 400x faster hashing", sections "BLAKE3" and "Merkle tree
 * reduction": every node of the tree is such a CV). When dev_in is the part of a larger
 * input that starts at chunk chunk_base and chunk_base is a multiple of the subtree's
 * size rounded up to a power of two, the result is that node of the larger input's
 * tree: shares of one input hashed on several devices combine through parent
 * compressions, and the two top subtrees are the root's message block.
 *   dev_in      device pointer, 16-byte aligned (may be NULL only if len == 0; len == 0 is
 *               the CV of one empty chunk).
 *   chunk_base  counter of the first chunk.
 *   key         host pointer to 8 key words (keyed mode), or NULL (default mode).
 *   dev_out32   device pointer to 32 writable bytes: the 8 CV words, little-endian.
 * Errors: EINVAL (NULL dev_out32, NULL dev_in with len > 0, chunk counter overflow),
 * EALIGN, ETOOBIG, ENOMEM, EHIP.
 */
int blake3_gpu_subtree_cv(const void *dev_in, uint64_t len, uint64_t chunk_base, const uint32_t key[8],
                          void *dev_out32, void *stream);

/*
 * Extendable output of dev_in[0 .. len): out_len bytes of the output stream of the
 * tree's root node, written to dev_out. Stream block t (64 bytes) is the root
 * compression run with counter t and ROOT, all sixteen output words (BLAKE3
 * specification, extendable output; the page lists it as future work, "Future work").
 * The first 32 bytes are the 32-byte hash; a longer request extends a shorter one.
 *   key         host pointer to 8 key words (keyed mode), or NULL (default mode).
 *   dev_out     device pointer to out_len writable bytes (any alignment).
 *   out_len     0 .. 2^42 bytes (0 enqueues nothing).
 * Other arguments and errors as blake3_gpu_hash (ETOOBIG also for out_len > 2^42).
 */
int blake3_gpu_hash_xof(const void *dev_in, uint64_t len, const uint32_t key[8], void *dev_out, uint64_t out_len,
                        void *stream);

/*
 * The same output stream read from any position: stream bytes [out_offset, out_offset +
 * out_len) of the extendable output of dev_in[0 .. len), written to dev_out[0 .. out_len)
 * (BLAKE3 specification, extendable output: block t of the stream depends only on t, so no
 * earlier block is computed). blake3_gpu_hash_xof is the case out_offset == 0. Useful for
 * consumers that each take a slice of one long output stream.
 *   out_offset  any byte offset; out_offset + out_len must not exceed 2^64 (the stream's
 *               last byte is byte 2^64 - 1).
 * Other arguments as blake3_gpu_hash_xof. Errors: as blake3_gpu_hash_xof, and EINVAL when
 * out_offset + out_len exceeds 2^64.
 */
int blake3_gpu_hash_xof_at(const void *dev_in, uint64_t len, const uint32_t key[8], uint64_t out_offset,
                           void *dev_out, uint64_t out_len, void *stream);

/*
 * The first tree level that one workgroup produces: the chaining value (CV) of every
 * aligned group of group_chunks consecutive 1 KiB chunks of dev_in[0 .. len) (the last
 * group may be shorter), with chunk counters starting at chunk_base and no ROOT flag
 * anywhere. This is the page's first kernel on its own ("Kernel 1": compress every chunk,
 * then a fused partial reduction to one root per block); each group CV is a node of the
 * BLAKE3 tree of any larger input of which dev_in is the part starting at chunk
 * chunk_base, provided chunk_base is a multiple of group_chunks. Uses: hashing an input
 * spread over several devices or produced piece by piece, and timing the chunk kernel
 * alone.
 *   dev_in       device pointer, 16-byte aligned, len > 0 bytes.
 *   chunk_base   counter of the first chunk of dev_in.
 *   key          host pointer to 8 key words (keyed mode), or NULL (default mode).
 *   group_chunks 64 (four lanes per chunk, the small-input leaf), 256, 512 or 1024
 *                (blake3_gpu_leaf_group_chunks(len) is what the hash entry points use for
 *                an input of len bytes).
 *   dev_cvs      device pointer, 16-byte aligned, to ceil(ceil(len/1024)/group_chunks) * 32
 *                bytes; group g's CV (8 little-endian words) at byte 32*g.
 * Errors: EINVAL (NULL dev_in or dev_cvs, len == 0, other group_chunks, counter
 * overflow), EALIGN, ETOOBIG (len above 2^42, or more groups than one launch holds:
 * 2^24 - 1, reached only above 2^40 bytes at 64 chunks per group and at 2^42 bytes at
 * 256), EHIP. Needs no scratch.
 */
int blake3_gpu_group_cvs(const void *dev_in, uint64_t len, uint64_t chunk_base, const uint32_t key[8],
                         uint32_t group_chunks, void *dev_cvs, void *stream);

/* Chunks per leaf workgroup that the hash entry points use for an input of len bytes: 64
 * for inputs of at most 32768 chunks (four lanes per chunk; the environment variable
 * BLAKE3_GPU_QUAD_LEAF_MAX_CHUNKS moves that bound), else 256, 512 or 1024 (larger
 * inputs fold more chunks per lane before the workgroup tree). An input of at most 2^15
 * chunks more than 2^16, 2^17 or 2^18 chunks is hashed as that power of two in groups of
 * 256, 512 or 1024 chunks (the value returned) and the chunks past it in groups of 64, in
 * one launch; the digest is the same for any grouping. */
uint32_t blake3_gpu_leaf_group_chunks(uint64_t len);

/* Static, human-readable text for a b3g_status value (never NULL). */
const char *blake3_gpu_strerror(int status);

/* Version of this ABI as major*10000 + minor*100 + patch. */
int blake3_gpu_version(void);

/*
 * Inspection of the batch planner, for tests and tools (no GPU work, no HIP call).
 * Plans the launches blake3_gpu_keyed_hash_batch makes for n messages of the given byte
 * lengths when the batch is not uniform, and serialises the plan into out[0 .. out_words)
 * as uint64 words:
 *   [passes] then per pass [lanes, chunks per lane K, workgroups W, segments S, in_cvs,
 *   out_cvs, W+1 first-segment indices, W level counts, S x (msg, first, dst, info)].
 * Segment info packs bits 0..11 lane start, 12..23 node count - 1, 30 pair, 31 final. In
 * pass 0 a node is a lane's run of K chunks and `first` a chunk index; later nodes are
 * CVs. Pair: the segment's last node is the parent of input CVs first + count - 1 and
 * first + count (the two halves of a message end that pass 0 split in two subtrees).
 * Returns the number of words the plan needs (nothing is written if out_words is
 * smaller), or a negative b3g_status (EINVAL for NULL lengths with n > 0, ETOOBIG).
 */
int64_t blake3_gpu_debug_plan_batch(const uint64_t *host_lengths, uint64_t n, uint64_t *out,
                                    uint64_t out_words);

/*
 * Test hooks. The library reads its BLAKE3_GPU_* environment variables (leaf and input-path
 * overrides, forced scratch failure and fill, and the like) once, when it is loaded, so no
 * call reads the environment. This reads them again, for tests and tools that change them
 * between calls; it must not run while another call of the library is running. No GPU
 * work, no HIP call. Returns B3G_OK.
 */
int blake3_gpu_debug_reload_env(void);

#ifdef __cplusplus
}
#endif

#endif /* BLAKE3_GPU_H */
