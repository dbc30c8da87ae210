/* Uses the library from C through include/blake3_gpu.h alone: device buffers from the HIP
 * runtime API, a stream of its own, every hashing entry point, and the results compared
 * with the CPU oracle (oracle/blake3_oracle.c, linked in for this check). Exit status 0
 * when every result matches. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "blake3_gpu.h"

/* the oracle's entry points used here */
void b3o_hash(const uint8_t *data, uint64_t len, uint8_t out32[32]);
void b3o_keyed_hash(const uint8_t *data, uint64_t len, const uint8_t key32[32], uint8_t out32[32]);
void b3o_hash_xof(const uint8_t *data, uint64_t len, const uint8_t *key32, uint8_t *out, uint64_t out_len);
void b3o_subtree_cv(const uint8_t *data, uint64_t len, uint64_t chunk_base, const uint8_t *key32, uint32_t out[8]);

#define CHECK_HIP(x)                                                     \
    do {                                                                 \
        if ((x) != hipSuccess) {                                         \
            fprintf(stderr, "HIP call failed at line %d\n", __LINE__); \
            return 2;                                                    \
        }                                                                \
    } while (0)

static int failures = 0;
static void expect(int ok, const char *what, uint64_t len) {
    if (!ok) {
        fprintf(stderr, "mismatch: %s, length %llu\n", what, (unsigned long long)len);
        ++failures;
    }
}

int main(void) {
    enum { N = 6 };
    const uint64_t lens[N] = {0, 1, 1024, 1025, 70000, (1u << 20) + 5};
    uint64_t offs[N], total = 0;
    for (int i = 0; i < N; ++i) {
        offs[i] = total;
        total += (lens[i] + 15) / 16 * 16;
    }
    uint8_t *host = (uint8_t *)malloc(total + 16);
    uint64_t s = 0x243F6A8885A308D3ull;
    for (uint64_t i = 0; i < total + 16; ++i) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        host[i] = (uint8_t)(s >> 56);
    }
    uint8_t keys[N][32];
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < 32; ++j) keys[i][j] = (uint8_t)(i * 37 + j * 11 + 5);

    void *d_in = NULL, *d_out = NULL, *d_keys = NULL, *d_batch = NULL;
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    CHECK_HIP(hipMalloc(&d_in, total + 16));
    CHECK_HIP(hipMalloc(&d_out, 4096));
    CHECK_HIP(hipMalloc(&d_keys, sizeof(keys)));
    CHECK_HIP(hipMalloc(&d_batch, 32 * N));
    CHECK_HIP(hipMemcpy(d_in, host, total + 16, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_keys, keys, sizeof(keys), hipMemcpyHostToDevice));

    for (int i = 0; i < N; ++i) {
        const uint8_t *msg = host + offs[i];
        const void *d_msg = (const uint8_t *)d_in + offs[i];
        uint32_t kw[8];
        memcpy(kw, keys[i], 32); /* little-endian words */
        uint8_t got[64], want[64];
        /* default mode */
        expect(blake3_gpu_hash(d_msg, lens[i], d_out, stream) == B3G_OK, "blake3_gpu_hash status", lens[i]);
        CHECK_HIP(hipMemcpyAsync(got, d_out, 32, hipMemcpyDeviceToHost, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        b3o_hash(msg, lens[i], want);
        expect(memcmp(got, want, 32) == 0, "blake3_gpu_hash", lens[i]);
        /* keyed mode */
        expect(blake3_gpu_keyed_hash(d_msg, lens[i], kw, d_out, stream) == B3G_OK, "keyed status", lens[i]);
        CHECK_HIP(hipMemcpyAsync(got, d_out, 32, hipMemcpyDeviceToHost, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        b3o_keyed_hash(msg, lens[i], keys[i], want);
        expect(memcmp(got, want, 32) == 0, "blake3_gpu_keyed_hash", lens[i]);
        /* extended output, 64 bytes */
        expect(blake3_gpu_hash_xof(d_msg, lens[i], kw, d_out, 64, stream) == B3G_OK, "xof status", lens[i]);
        CHECK_HIP(hipMemcpyAsync(got, d_out, 64, hipMemcpyDeviceToHost, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        b3o_hash_xof(msg, lens[i], keys[i], want, 64);
        expect(memcmp(got, want, 64) == 0, "blake3_gpu_hash_xof", lens[i]);
        /* subtree CV with a counter base above 2^32 */
        if (lens[i] > 0) {
            uint32_t cv[8], wcv[8];
            const uint64_t base = (1ull << 32) + 64;
            expect(blake3_gpu_subtree_cv(d_msg, lens[i], base, kw, d_out, stream) == B3G_OK, "subtree status",
                   lens[i]);
            CHECK_HIP(hipMemcpyAsync(cv, d_out, 32, hipMemcpyDeviceToHost, stream));
            CHECK_HIP(hipStreamSynchronize(stream));
            b3o_subtree_cv(msg, lens[i], base, keys[i], wcv);
            expect(memcmp(cv, wcv, 32) == 0, "blake3_gpu_subtree_cv", lens[i]);
        }
    }
    /* the same messages as one batch, one key each */
    uint8_t batch[N][32];
    expect(blake3_gpu_keyed_hash_batch(d_in, offs, lens, (const uint32_t *)d_keys, d_batch, N, stream) == B3G_OK,
           "batch status", N);
    CHECK_HIP(hipMemcpyAsync(batch, d_batch, sizeof(batch), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    for (int i = 0; i < N; ++i) {
        uint8_t want[32];
        b3o_keyed_hash(host + offs[i], lens[i], keys[i], want);
        expect(memcmp(batch[i], want, 32) == 0, "blake3_gpu_keyed_hash_batch", lens[i]);
    }
    /* argument errors are reported, not launched */
    expect(blake3_gpu_hash(NULL, 5, d_out, stream) == B3G_EINVAL, "EINVAL", 5);
    expect(blake3_gpu_hash((const uint8_t *)d_in + 4, 5, d_out, stream) == B3G_EALIGN, "EALIGN", 5);
    expect(blake3_gpu_strerror(B3G_EALIGN) != NULL && blake3_gpu_version() >= 10000, "strerror/version", 0);

    CHECK_HIP(hipFree(d_in));
    CHECK_HIP(hipFree(d_out));
    CHECK_HIP(hipFree(d_keys));
    CHECK_HIP(hipFree(d_batch));
    CHECK_HIP(hipStreamDestroy(stream));
    free(host);
    if (failures) return 1;
    puts("c abi: every result matches the oracle");
    return 0;
}
