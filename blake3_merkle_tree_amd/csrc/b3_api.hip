// b3_api.hip - the C ABI (include/blake3_gpu.h): argument checks, launch planning,
// scratch (library-owned slots, a stream-ordered pool), kernel launches.
//
// The chain of launches is the one of the page "BLAKE3 on GPU: 400x faster hashing"
// (qfminer.top), sections "Our implementation" and "Kernels 2 and 3": a leaf pass that
// compresses every chunk and reduces each workgroup's chunks to one chaining value,
// then level passes over those values until a single ROOT-flagged compression remains.
// All launches go to the caller's stream; nothing here waits for the device.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <memory>
#include <mutex>
#include <vector>

#include "blake3_gpu.h"
#include "b3_device.h"
#include "b3_kernels.h"
#include "b3_plan.h"

// Scratch of the entry point that allocates nothing (blake3_gpu_keyed_hash_noalloc): a fixed
// array of device memory. Each GPU the library runs on holds its own copy until the process
// ends, and every such call on that GPU uses it. In host code this name stands for a
// host-side shadow, not for device memory: the calling device's address of the array is
// looked up once per device (fixed_scratch_address) and only that address reaches kernels.
static __device__ __align__(256) uint8_t scratch[BLAKE3_GPU_NOALLOC_SCRATCH_BYTES];

namespace b3g {
namespace {

constexpr int kAbiVersion = 1 * 10000 + 3 * 100 + 0;

// Stream-ordered scratch comes from one memory pool per device, created on first use and
// kept for the life of the process, with a release threshold of "never" so that freed
// blocks are reused by the next call instead of being returned to the driver. Falls
// back to the device's default pool if a pool cannot be created.
constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pools[kMaxDevices] = {};
bool g_pool_tried[kMaxDevices] = {};

hipMemPool_t device_pool() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (!g_pool_tried[dev]) {
        g_pool_tried[dev] = true;
        hipMemPoolProps props{};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
            uint64_t keep = UINT64_MAX;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
            g_pools[dev] = pool;
        } else {
            (void)hipGetLastError();
        }
    }
    return g_pools[dev];
}

// Library-owned scratch slots, a few per device, each kept for the life of the process
// and grown when a call needs more. A call takes a slot that no other host thread holds,
// preferring one whose last use has finished on the device; its stream then waits on the
// slot's event (a device-side wait: the host does not block), and when the call has
// enqueued its work it records the slot's event on its stream. Calls on any streams thus
// use the memory one after another in the order in which they took it, without a
// stream-ordered allocation per call: such an allocation costs ~10 us of host time on an
// idle stream and ~100 us or more on a stream held behind long work, where the pool cannot
// reuse the block the same stream freed until the device has passed the free.
constexpr int kSlotsPerDevice = 4;
constexpr size_t kSlotMaxBytes = size_t(64) << 20;  // larger requests use the pool

// A scratch slot's event only marks when the device has passed the end of a call: the host
// tests it before it reuses the memory, and other streams wait on it on the device. None of
// that needs the system-scope cache write-back and invalidation that a recorded event
// otherwise performs, and which holds the next launch on the stream back by several
// microseconds. Every call records its events without it (MI355X, back to back, one
// process per build: 1 MiB 26.0 -> 23.9 us, 64 MiB 42.8 -> 40.5 us, 256 MiB 105.2 -> 103.1
// us; 256 ragged messages 74.1 -> 71.0 us with the task table's upload event unfenced too,
// 72.7 us with that one alone).
constexpr unsigned kUnfencedEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;
// Each slot also holds the tickets of fused level passes: zeroed once, when the slot's
// memory is allocated, and left at zero by every launch that uses them.
constexpr size_t kSlotTicketWords = 16384;

struct ScratchSlot {
    void *p = nullptr;
    size_t bytes = 0;
    uint32_t *tickets = nullptr;     // kSlotTicketWords words after the slot's `bytes`
    hipEvent_t done = nullptr;       // recorded after the work of the slot's last call (kUnfencedEventFlags)
    hipStream_t last = nullptr;      // that call's stream (a preference only: every reuse waits on done)
    bool used = false;               // done has been recorded
    bool held = false;               // taken by a call that has not yet returned
};
struct DeviceSlots {
    std::mutex mu;
    ScratchSlot slot[kSlotsPerDevice];
    // Memory of slots that outgrew it. It is never freed: hipFree waits for every stream of
    // the device, and a call must not. A slot grows in powers of two up to kSlotMaxBytes,
    // so what is kept this way stays below that per slot.
    std::vector<void *> retired;
};
DeviceSlots g_slots[kMaxDevices];

// Test hook: with BLAKE3_GPU_SCRATCH_FILL set, a call's scratch is filled with that byte
// before its kernels run (by a kernel in stream order), so that tests can show that no
// result depends on what the memory held before. Scratch requests are multiples of 4 bytes.
int fill_scratch(void *p, size_t bytes, hipStream_t s) {
    const int fill = scratch_fill_byte();
    if (fill < 0) return B3G_OK;
    const uint32_t word = 0x01010101u * static_cast<uint32_t>(fill);
    if (launch_fill_words(static_cast<uint32_t *>(p), word, bytes / 4, s) != hipSuccess) {
        (void)hipGetLastError();
        return B3G_EHIP;
    }
    return B3G_OK;
}

// Scratch of one call: a slot (above), or, for large requests or when every slot is held,
// a stream-ordered allocation released in stream order on the caller's stream.
class StreamScratch {
  public:
    explicit StreamScratch(hipStream_t s) : s_(s) {}
    ~StreamScratch() {
        if (slot_ != nullptr) {
            std::lock_guard<std::mutex> lock(slots_->mu);
            if (hipEventRecord(slot_->done, s_) != hipSuccess) {
                // the device could not be told when this call's work ends: never reuse the memory
                (void)hipGetLastError();
                slot_->p = nullptr;
                slot_->bytes = 0;
                slot_->used = false;
            } else {
                slot_->last = s_;
                slot_->used = true;
            }
            slot_->held = false;
        } else if (p_) {
            (void)hipFreeAsync(p_, s_);
        }
    }
    int alloc(size_t bytes) {
        if (bytes == 0) return B3G_OK;
        if (bytes > scratch_limit()) return B3G_ENOMEM;  // test hook: a forced allocation failure
        int rc = bytes <= kSlotMaxBytes ? take_slot(bytes) : B3G_ENOMEM;
        if (rc != B3G_OK) rc = from_pool(bytes);
        if (rc != B3G_OK) return rc;
        return fill_scratch(p_, bytes, s_);
    }
    uint8_t *get() const { return static_cast<uint8_t *>(p_); }
    // Zeroed tickets of the slot this call holds (left at zero by every launch that uses
    // them), or nullptr: scratch from the pool, or more tickets than a slot holds.
    uint32_t *zeroed_tickets(size_t words) const {
        return slot_ != nullptr && words <= kSlotTicketWords ? slot_->tickets : nullptr;
    }

  private:
    int take_slot(size_t bytes) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
            (void)hipGetLastError();
            return B3G_ENOMEM;
        }
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s_, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
            (void)hipGetLastError();
            return B3G_ENOMEM;  // under graph capture: the stream-ordered pool, as recorded nodes
        }
        DeviceSlots &ds = g_slots[dev];
        ScratchSlot *sl = nullptr;
        bool wait = false;
        {
            std::lock_guard<std::mutex> lock(ds.mu);
            // Preference: large enough and idle on the device (4); large enough and last used
            // on this stream, so that waiting for it costs nothing (3); idle but too small, to
            // be grown (2); large enough but in use on another stream, a device-side wait (1).
            // A slot still in use and too small is never taken: growing it would block the host.
            int best = -1, score = 0;
            for (int i = 0; i < kSlotsPerDevice; ++i) {
                ScratchSlot &c = ds.slot[i];
                if (c.held) continue;
                bool idle = !c.used;
                if (!idle) {
                    idle = hipEventQuery(c.done) == hipSuccess;
                    if (!idle) (void)hipGetLastError();  // not ready yet
                }
                const bool fits = c.bytes >= bytes;
                const int sc = fits ? (idle ? 4 : (c.last == s_ ? 3 : 1)) : (idle ? 2 : 0);
                if (sc > score) {
                    best = i;
                    score = sc;
                }
            }
            if (best < 0) return B3G_ENOMEM;  // the pool instead
            sl = &ds.slot[best];
            sl->held = true;
            // a slot last used on this stream needs no wait: the stream's order holds
            wait = sl->used && score == 1;
        }
        if (sl->done == nullptr && hipEventCreateWithFlags(&sl->done, kUnfencedEventFlags) != hipSuccess) {
            (void)hipGetLastError();
            sl->done = nullptr;
            return release_unused(ds, sl);
        }
        if (sl->bytes < bytes) {  // grow an idle slot (its last call's work has finished)
            if (sl->p != nullptr) {
                std::lock_guard<std::mutex> lock(ds.mu);
                ds.retired.push_back(sl->p);
            }
            sl->p = nullptr;
            sl->bytes = 0;
            size_t grown = size_t(1) << 20;
            while (grown < bytes) grown <<= 1;
            if (hipMalloc(&sl->p, grown + kSlotTicketWords * 4) != hipSuccess) {
                (void)hipGetLastError();
                sl->p = nullptr;
                return release_unused(ds, sl);
            }
            sl->tickets = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(sl->p) + grown);
            // zero the tickets in stream order, before this call's kernels (a slot that is
            // grown is idle: no launch still uses its old memory)
            if (launch_fill_words(sl->tickets, 0, kSlotTicketWords, s_) != hipSuccess) {
                (void)hipGetLastError();
                std::lock_guard<std::mutex> lock(ds.mu);
                ds.retired.push_back(sl->p);
                sl->p = nullptr;
                sl->tickets = nullptr;
                sl->held = false;
                return B3G_ENOMEM;
            }
            sl->bytes = grown;
        } else if (wait && hipStreamWaitEvent(s_, sl->done, 0) != hipSuccess) {  // after its last call
            (void)hipGetLastError();
            return release_unused(ds, sl);
        }
        slot_ = sl;
        slots_ = &ds;
        p_ = sl->p;
        return B3G_OK;
    }
    static int release_unused(DeviceSlots &ds, ScratchSlot *sl) {
        std::lock_guard<std::mutex> lock(ds.mu);
        sl->held = false;
        return B3G_ENOMEM;
    }
    int from_pool(size_t bytes) {
        hipMemPool_t pool = device_pool();
        const hipError_t e = pool ? hipMallocFromPoolAsync(&p_, bytes, pool, s_) : hipMallocAsync(&p_, bytes, s_);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            p_ = nullptr;
            return B3G_ENOMEM;
        }
        return B3G_OK;
    }

    hipStream_t s_;
    void *p_ = nullptr;
    ScratchSlot *slot_ = nullptr;
    DeviceSlots *slots_ = nullptr;
};

// Device address of `scratch` per device, looked up on the device's first no-allocation
// call (with that device current) and kept.
std::mutex g_fixed_mu;
std::atomic<uint8_t *> g_fixed_ptr[kMaxDevices];

int fixed_scratch_address(uint8_t **p) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return B3G_EHIP;
    }
    uint8_t *q = g_fixed_ptr[dev].load(std::memory_order_acquire);
    if (q == nullptr) {
        std::lock_guard<std::mutex> lock(g_fixed_mu);
        q = g_fixed_ptr[dev].load(std::memory_order_relaxed);
        if (q == nullptr) {
            void *addr = nullptr;
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
                (void)hipGetLastError();
                return B3G_EHIP;
            }
            q = static_cast<uint8_t *>(addr);
            g_fixed_ptr[dev].store(q, std::memory_order_release);
        }
    }
    *p = q;
    return B3G_OK;
}

// Scratch of one hash: a slot or the pool (StreamScratch), or, for the entry point that
// allocates nothing, the calling device's copy of the fixed array. A request larger than
// that array fails with B3G_ESCRATCH before any HIP call.
class CallScratch {
  public:
    CallScratch(hipStream_t s, bool fixed) : s_(s), fixed_(fixed), pooled_(s) {}
    int alloc(size_t bytes) {
        if (!fixed_) {
            const int rc = pooled_.alloc(bytes);
            p_ = pooled_.get();
            return rc;
        }
        if (bytes > BLAKE3_GPU_NOALLOC_SCRATCH_BYTES) return B3G_ESCRATCH;
        if (bytes == 0) return B3G_OK;
        const int rc = fixed_scratch_address(&p_);
        if (rc != B3G_OK) return rc;
        return fill_scratch(p_, bytes, s_);
    }
    uint8_t *get() const { return p_; }
    uint32_t *zeroed_tickets(size_t words) const { return fixed_ ? nullptr : pooled_.zeroed_tickets(words); }

  private:
    hipStream_t s_;
    bool fixed_;
    StreamScratch pooled_;  // unused (never allocates) when fixed_
    uint8_t *p_ = nullptr;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int launched(hipError_t e) {
    if (e == hipSuccess) return B3G_OK;
    (void)hipGetLastError();
    return B3G_EHIP;
}

// Pinned host buffers for the batch task tables, up to 16 per device, allocated on first use
// (coherent, device-visible), grown when needed and kept. A table is built in one and
// uploaded by a copy kernel on the caller's stream, which reads it over the bus: the
// kernels after it wait for nothing but the stream's order, where a copy-engine transfer
// from pageable memory left ~18 us between a batch's launches. The buffer's event,
// recorded after that kernel (without the system-scope fence: it only has to show that the
// kernel's reads are done), must have completed before the host writes the buffer again. A call that finds no such buffer free builds its table in pageable memory and
// copies it with hipMemcpyAsync: the host never waits for the device here.
constexpr int kStagesPerDevice = 16;
constexpr size_t kStageArenaSlice = size_t(256) << 10;  // each buffer's first size, from one arena
constexpr size_t kStageMaxBytes = size_t(64) << 20;

struct HostStage {
    void *p = nullptr;          // host address
    void *dev = nullptr;        // the same memory as the device addresses it
    size_t bytes = 0;
    hipEvent_t done = nullptr;  // recorded after the last upload from this buffer
    bool own = false;           // allocated on its own (else a slice of the arena)
    bool used = false;
    bool held = false;
};
struct DeviceStages {
    std::mutex mu;
    bool arena_tried = false;  // one pinned allocation for every buffer's first size, made once
    HostStage stage[kStagesPerDevice];
    // Buffers that were outgrown. Never freed: hipHostFree waits for every stream of the
    // device, and a call must not.
    std::vector<void *> retired;
};
DeviceStages g_stages[kMaxDevices];

class TableStage {
  public:
    ~TableStage() {
        if (st_ != nullptr) {
            std::lock_guard<std::mutex> lock(ds_->mu);
            st_->held = false;
        }
    }
    // A pinned buffer of at least `bytes` that no upload still reads, or nullptr.
    uint8_t *take(size_t bytes) {
        int dev = 0;
        if (bytes == 0 || bytes > kStageMaxBytes || hipGetDevice(&dev) != hipSuccess || dev < 0 ||
            dev >= kMaxDevices) {
            (void)hipGetLastError();
            return nullptr;
        }
        DeviceStages &ds = g_stages[dev];
        HostStage *st = nullptr;
        {
            std::lock_guard<std::mutex> lock(ds.mu);
            if (!ds.arena_tried) {
                ds.arena_tried = true;
                void *a = nullptr, *da = nullptr;
                if (hipHostMalloc(&a, kStagesPerDevice * kStageArenaSlice, hipHostMallocCoherent) == hipSuccess &&
                    hipHostGetDevicePointer(&da, a, 0) == hipSuccess && da != nullptr) {
                    for (int i = 0; i < kStagesPerDevice; ++i) {
                        ds.stage[i].p = static_cast<uint8_t *>(a) + i * kStageArenaSlice;
                        ds.stage[i].dev = static_cast<uint8_t *>(da) + i * kStageArenaSlice;
                        ds.stage[i].bytes = kStageArenaSlice;
                    }
                } else {
                    (void)hipGetLastError();
                    if (a != nullptr) ds.retired.push_back(a);  // unusable; freeing it would wait for the device
                }
            }
            int best = -1;
            for (int i = 0; i < kStagesPerDevice; ++i) {
                HostStage &c = ds.stage[i];
                if (c.held) continue;
                if (c.used && hipEventQuery(c.done) != hipSuccess) {
                    (void)hipGetLastError();  // an upload still reads it
                    continue;
                }
                // idle: the smallest that fits, else the largest (to grow)
                if (best < 0) {
                    best = i;
                    continue;
                }
                const HostStage &b = ds.stage[best];
                const bool cf = c.bytes >= bytes, bf = b.bytes >= bytes;
                if ((cf && (!bf || c.bytes < b.bytes)) || (!cf && !bf && c.bytes > b.bytes)) best = i;
            }
            if (best < 0) return nullptr;
            st = &ds.stage[best];
            st->held = true;
        }
        st_ = st;
        ds_ = &ds;
        if (st->done == nullptr && hipEventCreateWithFlags(&st->done, kUnfencedEventFlags) != hipSuccess) {
            (void)hipGetLastError();
            st->done = nullptr;
            return release();
        }
        if (st->bytes < bytes) {
            if (st->own) {  // idle (no upload reads it), but freeing it would wait for the device
                std::lock_guard<std::mutex> lock(ds.mu);
                ds.retired.push_back(st->p);
            }
            st->p = st->dev = nullptr;
            st->bytes = 0;
            st->own = false;
            size_t grown = kStageArenaSlice;
            while (grown < bytes) grown <<= 1;
            void *p = nullptr, *dp = nullptr;
            if (hipHostMalloc(&p, grown, hipHostMallocCoherent) != hipSuccess) {
                (void)hipGetLastError();
                return release();
            }
            if (hipHostGetDevicePointer(&dp, p, 0) != hipSuccess || dp == nullptr) {
                (void)hipGetLastError();
                std::lock_guard<std::mutex> lock(ds.mu);
                ds.retired.push_back(p);  // unusable, and freeing it would wait for the device
                return release();
            }
            st->p = p;
            st->dev = dp;
            st->bytes = grown;
            st->own = true;
        }
        return static_cast<uint8_t *>(st->p);
    }
    // Uploads the first `bytes` (a multiple of 16) of the buffer to dst on s. The buffer's
    // event is recorded right after the copy, so that the buffer is free again as soon as the
    // copy has run (the host may be many calls ahead of the device).
    int upload(void *dst, size_t bytes, hipStream_t s) {
        const int rc = launched(launch_copy_words16(st_->dev, dst, bytes / 16, s));
        if (rc != B3G_OK) return rc;
        std::lock_guard<std::mutex> lock(ds_->mu);
        if (hipEventRecord(st_->done, s) == hipSuccess) {
            st_->used = true;
        } else {  // unknown when the upload ends: never write this buffer again
            (void)hipGetLastError();
            st_->p = st_->dev = nullptr;
            st_->bytes = 0;
            st_->own = false;
            st_->used = false;
        }
        return B3G_OK;
    }

  private:
    uint8_t *release() {
        std::lock_guard<std::mutex> lock(ds_->mu);
        st_->held = false;
        st_ = nullptr;
        return nullptr;
    }
    HostStage *st_ = nullptr;
    DeviceStages *ds_ = nullptr;
};

uint32_t next_pow2_u32(uint64_t x) {
    uint32_t r = 1;
    while (r < x) r <<= 1;
    return r;
}

// Largest grid of one launch: HIP caps a grid at 2^32 - 1 work-items.
constexpr uint64_t kMaxGrid = 0xFFFFFFFFull / kLeafLanes;

// One message of len bytes whose chunk count is a little above T0 = 2^16 * k (see
// split_tail_chunks_per_lane): its first T0 chunks as 256 leaf workgroups of 256 * k chunks
// and the rest on quad workgroups, in one launch (leaf_split_kernel), then both subtrees and
// their parent in one workgroup (level_split_root_kernel). out receives the root digest, or
// with root_flag 0 the message's CV.
int hash_split(const uint8_t *base, uint64_t len, const uint32_t key[8], uint32_t mode, uint64_t chunk_base,
               uint32_t root_flag, uint8_t *out, uint32_t k, hipStream_t s, bool fixed) {
    const uint64_t t0 = (1ull << 16) * k;
    const uint64_t tail_chunks = chunks_of(len) - t0;
    const uint32_t tail_wgs = static_cast<uint32_t>((tail_chunks + kQuadLeafChunks - 1) / kQuadLeafChunks);
    CallScratch scratch(s, fixed);
    int rc = scratch.alloc(static_cast<size_t>(kLevelLanes + tail_wgs) * 32);
    if (rc != B3G_OK) return rc;
    auto *cvs = reinterpret_cast<uint32_t *>(scratch.get());

    SplitLeafArgs a{};
    UniformLeafArgs &m = a.main;  // case B: 256 groups of 256 * k whole chunks
    m.base = base;
    m.len = t0 * kChunkBytes;
    m.n_chunks = t0;
    m.chunk_base = chunk_base;
    m.n_msgs = 1;
    m.groups = kLevelLanes;
    memcpy(m.key, key, sizeof(m.key));
    m.mode = mode;
    m.cv_out = cvs;
    UniformLeafArgs &t = a.tail;  // case B on quads: tail_wgs groups of 64 chunks
    t = m;
    t.base = base + t0 * kChunkBytes;
    t.len = len - t0 * kChunkBytes;
    t.n_chunks = tail_chunks;
    t.chunk_base = chunk_base + t0;
    t.groups = tail_wgs;
    t.cv_out = cvs + 8ull * kLevelLanes;
    a.tail_wgs = tail_wgs;
    rc = launched(launch_split_leaf(a, k, s));
    if (rc != B3G_OK) return rc;

    SplitRootArgs r{};
    r.main_cv = cvs;
    r.tail_cv = cvs + 8ull * kLevelLanes;
    r.tail_n = tail_wgs;
    memcpy(r.key, key, sizeof(r.key));
    r.mode = mode;
    r.root_flag = root_flag;
    r.out = out;
    return launched(launch_split_root(r, s));
}

// n_msgs messages of len bytes each, message m at base + m * stride (wrapping 64-bit
// arithmetic), keyed by keys + 8*m (device) or all by `key` (host words). A leaf
// workgroup covers `span` chunks (256*K, or 64 with the quad leaf for small inputs). A
// message of at most `span` chunks is finished by the leaf pass, span/R messages per
// workgroup. A longer one spans G leaf workgroups, whose CVs the level passes reduce,
// 256 to a workgroup, until at most 256 remain, which one last pass finishes. Pass
// outputs ping-pong between two CV arrays, in scratch from the slots or the pool, or, with
// `fixed`, in the fixed array (nothing is allocated).
int hash_uniform(const uint8_t *base, uint64_t stride, uint64_t len, uint64_t n_msgs, const uint32_t *keys,
                 const uint32_t key[8], uint32_t mode, uint64_t chunk_base, uint32_t root_flag, uint8_t *out,
                 hipStream_t s, bool fixed = false) {
    if (n_msgs == 0) return B3G_OK;
    const uint64_t c = chunks_of(len);
    if (n_msgs == 1 && keys == nullptr && !fuse_uniform_levels() && !use_lds_staging()) {
        if (const uint32_t ks = split_tail_chunks_per_lane(c))
            return hash_split(base, len, key, mode, chunk_base, root_flag, out, ks, s, fixed);
    }
    const uint64_t total = c > UINT64_MAX / n_msgs ? UINT64_MAX : c * n_msgs;  // chunks, saturated
    // small inputs: a quad per chunk, kQuadLeafChunks chunk slots per workgroup
    const bool quad = total <= quad_leaf_max_chunks();
    uint32_t k = n_msgs == 1 ? choose_single_chunks_per_lane(total) : choose_chunks_per_lane(total);
    while (k > 1 && k > c) k >>= 1;  // a lane's run of chunks does not outgrow the message
    if (quad) k = 1;
    const uint64_t span = quad ? kQuadLeafChunks : static_cast<uint64_t>(kLeafLanes) * k;
    const uint32_t wg_slots = quad ? kQuadLeafChunks : kLeafLanes;  // nodes per leaf workgroup
    const bool fused = fuse_uniform_levels();
    const bool staged = use_lds_staging() && !fused;  // the fused leaf loads directly
    auto leaf = [&](const UniformLeafArgs &args, uint32_t grid) {
        return quad ? launch_quad_leaf(args, grid, s) : launch_uniform_leaf(args, k, staged, grid, s);
    };

    UniformLeafArgs la{};
    la.stride = stride;
    la.len = len;
    la.n_chunks = c;
    la.chunk_base = chunk_base;
    la.may_root = 1;
    la.root_flag = root_flag;
    la.keys = keys;
    memcpy(la.key, key, sizeof(la.key));
    la.mode = mode;

    if (c <= span) {  // case A: every message is finished by its leaf workgroup
        const uint32_t r = next_pow2_u32((c + k - 1) / k);
        const uint64_t per_wg = wg_slots / r;
        for (uint64_t m0 = 0; m0 < n_msgs; m0 += kMaxGrid * per_wg) {
            const uint64_t nm = n_msgs - m0 < kMaxGrid * per_wg ? n_msgs - m0 : kMaxGrid * per_wg;
            la.base = base + m0 * stride;
            la.n_msgs = static_cast<uint32_t>(nm);
            la.lanes_per_msg = r;
            la.groups = 1;
            la.keys = keys ? keys + 8 * m0 : nullptr;
            la.digests = out + 32 * m0;
            const int rc = launched(leaf(la, static_cast<uint32_t>((nm + per_wg - 1) / per_wg)));
            if (rc != B3G_OK) return rc;
        }
        return B3G_OK;
    }

    // case B: G = ceil(c / span) leaf workgroups per message
    const uint64_t g = (c + span - 1) / span;
    // one message's workgroups go in one launch. From 2^21 chunks a workgroup covers 1024
    // chunks, so at 2^42 bytes g is at most 2^22; only a leaf forced by a test hook onto a
    // huge input (the quad leaf, or one chunk per lane at 2^42 bytes) needs more
    if (g > kMaxGrid) return B3G_ETOOBIG;
    const uint64_t per_launch = kMaxGrid / g;  // >= 1
    const uint64_t nb = n_msgs < per_launch ? n_msgs : per_launch;
    const uint64_t g1 = (g + kLevelLanes - 1) / kLevelLanes;
    CallScratch scratch(s, fixed);

    if (fused) {
        // One launch: the leaf workgroups reduce the levels themselves (last arrival of
        // each group of 256 takes it up a level). Scratch: the CVs of every level but the
        // root, and one zeroed ticket per group above the leaf.
        uint64_t lg[kMaxLevels + 1] = {g, 0, 0, 0, 0};
        uint32_t levels = 0;
        while (lg[levels] > 1) {
            if (levels == kMaxLevels) return B3G_ETOOBIG;
            lg[levels + 1] = (lg[levels] + kLevelLanes - 1) / kLevelLanes;
            ++levels;
        }
        size_t cv_at[kMaxLevels], ctr_at[kMaxLevels], at = 0, ctr_words = 0;
        for (uint32_t L = 0; L < levels; ++L) {
            cv_at[L] = at;
            at += align256(nb * lg[L] * 32);
        }
        for (uint32_t L = 0; L < levels; ++L) {
            ctr_at[L] = ctr_words;
            ctr_words += nb * lg[L + 1];
        }
        // tickets: the slot's (zero, and left at zero by every launch), else zeroed by a
        // fill kernel before each launch, after the CVs in this call's scratch
        const size_t cv_bytes = at;
        int rc = scratch.alloc(cv_bytes + align256(ctr_words * 4));
        if (rc != B3G_OK) return rc;
        uint8_t *d = scratch.get();
        uint32_t *tickets = scratch.zeroed_tickets(ctr_words);
        const bool fill_tickets = tickets == nullptr;
        if (fill_tickets) tickets = reinterpret_cast<uint32_t *>(d + cv_bytes);
        la.levels = levels;
        for (uint32_t L = 0; L < levels; ++L) {
            la.lvl_cv[L] = reinterpret_cast<uint32_t *>(d + cv_at[L]);
            la.lvl_ctr[L] = tickets + ctr_at[L];
        }
        for (uint32_t L = 0; L <= levels; ++L) la.lvl_g[L] = lg[L];
        for (uint64_t m0 = 0; m0 < n_msgs; m0 += nb) {
            const uint64_t nm = n_msgs - m0 < nb ? n_msgs - m0 : nb;
            if (fill_tickets) {
                rc = launched(launch_zero_words(tickets, ctr_words, s));
                if (rc != B3G_OK) return rc;
            }
            la.base = base + m0 * stride;
            la.n_msgs = static_cast<uint32_t>(nm);
            la.lanes_per_msg = 0;
            la.groups = static_cast<uint32_t>(g);
            la.keys = keys ? keys + 8 * m0 : nullptr;
            la.cv_out = la.lvl_cv[0];
            la.digests = out + 32 * m0;
            rc = launched(leaf(la, static_cast<uint32_t>(nm * g)));
            if (rc != B3G_OK) return rc;
        }
        return B3G_OK;
    }

    const size_t a_bytes = align256(nb * g * 32);
    int rc = scratch.alloc(a_bytes + (g1 > 1 ? align256(nb * g1 * 32) : 0));
    if (rc != B3G_OK) return rc;
    uint32_t *cv_a = reinterpret_cast<uint32_t *>(scratch.get());
    uint32_t *cv_b = reinterpret_cast<uint32_t *>(scratch.get() + a_bytes);

    for (uint64_t m0 = 0; m0 < n_msgs; m0 += nb) {
        const uint64_t nm = n_msgs - m0 < nb ? n_msgs - m0 : nb;
        const uint32_t *mkeys = keys ? keys + 8 * m0 : nullptr;
        la.base = base + m0 * stride;
        la.n_msgs = static_cast<uint32_t>(nm);
        la.lanes_per_msg = 0;
        la.groups = static_cast<uint32_t>(g);
        la.keys = mkeys;
        la.cv_out = cv_a;
        la.digests = nullptr;
        rc = launched(leaf(la, static_cast<uint32_t>(nm * g)));
        if (rc != B3G_OK) return rc;

        uint64_t m = g;
        const uint32_t *src = cv_a;
        uint32_t *dst = cv_b;
        for (;;) {
            UniformLevelArgs lv{};
            lv.cv_in = src;
            lv.g_in = m;
            lv.n_msgs = static_cast<uint32_t>(nm);
            lv.keys = mkeys;
            memcpy(lv.key, key, sizeof(lv.key));
            lv.mode = mode;
            lv.root_flag = root_flag;
            if (m <= kLevelLanes) {  // last pass: 256/R messages per workgroup, digests out
                const uint32_t r = next_pow2_u32(m);
                const uint64_t per_wg = kLevelLanes / r;
                lv.lanes_per_msg = r;
                lv.digests = out + 32 * m0;
                rc = launched(launch_uniform_level(lv, static_cast<uint32_t>((nm + per_wg - 1) / per_wg), s));
                if (rc != B3G_OK) return rc;
                break;
            }
            const uint64_t w = (m + kLevelLanes - 1) / kLevelLanes;
            lv.lanes_per_msg = 0;
            lv.g_out = static_cast<uint32_t>(w);
            lv.cv_out = dst;
            rc = launched(launch_uniform_level(lv, static_cast<uint32_t>(nm * w), s));
            if (rc != B3G_OK) return rc;
            m = w;
            uint32_t *next_dst = const_cast<uint32_t *>(src);
            src = dst;
            dst = next_dst;
        }
    }
    return B3G_OK;
}

int hash_single(const void *in, uint64_t len, const uint32_t key[8], uint32_t mode, void *out, void *stream,
                bool fixed = false) {
    if (out == nullptr || (in == nullptr && len > 0)) return B3G_EINVAL;
    if (reinterpret_cast<uintptr_t>(in) % 16 != 0) return B3G_EALIGN;
    if (len > kMaxMessageBytes) return B3G_ETOOBIG;
    return hash_uniform(static_cast<const uint8_t *>(in), 0, len, 1, nullptr, key, mode, 0, kRoot,
                        static_cast<uint8_t *>(out), static_cast<hipStream_t>(stream), fixed);
}

// The CV (no ROOT) of the subtree over all chunks of in[0 .. len), chunk counters from
// chunk_base: the whole-message path with the top flag left out.
int subtree_cv(const void *in, uint64_t len, uint64_t chunk_base, const uint32_t *key, void *out, void *stream) {
    if (out == nullptr || (in == nullptr && len > 0)) return B3G_EINVAL;
    if (reinterpret_cast<uintptr_t>(in) % 16 != 0) return B3G_EALIGN;
    if (len > kMaxMessageBytes) return B3G_ETOOBIG;
    if (chunk_base + chunks_of(len) < chunk_base) return B3G_EINVAL;
    return hash_uniform(static_cast<const uint8_t *>(in), 0, len, 1, nullptr, key ? key : kIV,
                        key ? kKeyedHash : 0u, chunk_base, 0u, static_cast<uint8_t *>(out),
                        static_cast<hipStream_t>(stream));
}

// Extended output. The root node's inputs are gathered first: for one chunk, a small
// kernel chains the chunk's blocks up to the last one and copies the last block; for
// more, the two top subtrees (left: the largest power of two of chunks below n) are
// hashed without ROOT into one 64-byte block. Then every output block t is the root
// compression with counter t, one lane each; out receives stream bytes
// [out_offset, out_offset + out_len).
int hash_xof(const void *in, uint64_t len, const uint32_t *key, uint64_t out_offset, void *out, uint64_t out_len,
             void *stream) {
    if ((out == nullptr && out_len > 0) || (in == nullptr && len > 0)) return B3G_EINVAL;
    // the stream is 2^64 bytes: the request may end at byte 2^64, not beyond
    if (out_len > 0 && out_len - 1 > UINT64_MAX - out_offset) return B3G_EINVAL;
    if (reinterpret_cast<uintptr_t>(in) % 16 != 0) return B3G_EALIGN;
    if (len > kMaxMessageBytes || out_len > kMaxXofBytes) return B3G_ETOOBIG;
    if (out_len == 0) return B3G_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t *kw = key ? key : kIV;
    const uint32_t mode = key ? kKeyedHash : 0u;

    StreamScratch scratch(s);
    int rc = scratch.alloc(256);
    if (rc != B3G_OK) return rc;
    auto *rec_m = reinterpret_cast<uint32_t *>(scratch.get());       // 16 message words
    auto *rec_cv = reinterpret_cast<uint32_t *>(scratch.get() + 64);  // 8 CV words (one chunk)

    XofArgs x{};
    memcpy(x.key, kw, sizeof(x.key));
    x.m = rec_m;
    x.out = static_cast<uint8_t *>(out);
    x.out_offset = out_offset;
    x.out_len = out_len;
    const uint64_t n = chunks_of(len);
    if (n == 1) {
        const uint64_t nb = len == 0 ? 1 : (len + kBlockBytes - 1) / kBlockBytes;
        ChunkRootArgs c{static_cast<const uint8_t *>(in), static_cast<uint32_t>(len), {}, mode, rec_cv, rec_m};
        memcpy(c.key, kw, sizeof(c.key));
        rc = launched(launch_xof_chunk_root(c, s));
        if (rc != B3G_OK) return rc;
        x.cv = rec_cv;
        x.block_len = static_cast<uint32_t>(len - kBlockBytes * (nb - 1));
        x.flags = mode | kChunkEnd | (nb == 1 ? kChunkStart : 0u) | kRoot;
    } else {
        uint64_t k = 1;
        while (k * 2 < n) k *= 2;
        const uint8_t *bytes = static_cast<const uint8_t *>(in);
        rc = hash_uniform(bytes, 0, k * kChunkBytes, 1, nullptr, kw, mode, 0, 0u,
                          reinterpret_cast<uint8_t *>(rec_m), s);
        if (rc != B3G_OK) return rc;
        rc = hash_uniform(bytes + k * kChunkBytes, 0, len - k * kChunkBytes, 1, nullptr, kw, mode, k, 0u,
                          reinterpret_cast<uint8_t *>(rec_m + 8), s);
        if (rc != B3G_OK) return rc;
        x.cv = nullptr;  // the key words
        x.block_len = kBlockBytes;
        x.flags = mode | kParent | kRoot;
    }
    // blocks first_b .. end_b - 1, in launches that never cross a multiple of 2^32 blocks
    const uint64_t first_b = out_offset / kBlockBytes;
    const uint64_t last_byte = out_offset + out_len - 1;
    const uint64_t end_b = last_byte / kBlockBytes + 1;
    constexpr uint64_t kPerLaunch = kMaxGrid * kXofLanes;
    for (uint64_t b0 = first_b; b0 < end_b;) {
        const uint64_t to_wrap = (1ull << 32) - (b0 & 0xFFFFFFFFull);
        uint64_t nblk = end_b - b0;
        if (nblk > kPerLaunch) nblk = kPerLaunch;
        if (nblk > to_wrap) nblk = to_wrap;
        x.first_block = b0;
        x.n_blocks = nblk;
        rc = launched(launch_xof_expand(x, static_cast<uint32_t>((nblk + kXofLanes - 1) / kXofLanes), s));
        if (rc != B3G_OK) return rc;
        b0 += nblk;
    }
    return B3G_OK;
}

// Leaf pass only: the CV of every aligned group of group_chunks (= kLeafLanes * K)
// chunks, chunk counters starting at chunk_base, no ROOT anywhere.
int group_cvs(const void *in, uint64_t len, uint64_t chunk_base, const uint32_t *key, uint32_t group_chunks,
              void *out, void *stream) {
    if (out == nullptr || len == 0 || in == nullptr) return B3G_EINVAL;
    const bool quad = group_chunks == kQuadLeafChunks;
    if (!quad && group_chunks != kLeafLanes && group_chunks != 2 * kLeafLanes && group_chunks != 4 * kLeafLanes)
        return B3G_EINVAL;
    if (reinterpret_cast<uintptr_t>(in) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return B3G_EALIGN;
    if (len > kMaxMessageBytes) return B3G_ETOOBIG;
    const uint64_t n = chunks_of(len);
    if (chunk_base + n < chunk_base) return B3G_EINVAL;
    UniformLeafArgs la{};
    la.base = static_cast<const uint8_t *>(in);
    la.stride = 0;
    la.len = len;
    la.n_chunks = n;
    la.chunk_base = chunk_base;
    la.n_msgs = 1;
    la.lanes_per_msg = 0;
    const uint64_t groups = (n + group_chunks - 1) / group_chunks;
    if (groups > kMaxGrid) return B3G_ETOOBIG;  // one launch: at most 2^32 - 1 work-items
    la.groups = static_cast<uint32_t>(groups);
    la.may_root = 0;
    la.keys = nullptr;
    if (key) memcpy(la.key, key, sizeof(la.key));
    else memcpy(la.key, kIV, sizeof(la.key));
    la.mode = key ? kKeyedHash : 0u;
    la.cv_out = static_cast<uint32_t *>(out);
    la.digests = nullptr;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (quad) return launched(launch_quad_leaf(la, la.groups, s));
    return launched(launch_uniform_leaf(la, group_chunks / kLeafLanes, use_lds_staging(), la.groups, s));
}

template <class T>
void copy_bytes(uint8_t *img, size_t at, const std::vector<T> &v) {
    if (!v.empty()) memcpy(img + at, v.data(), v.size() * sizeof(T));
}

int hash_batch(const void *base, const uint64_t *offsets, const uint64_t *lengths, const uint32_t *keys,
               void *out, uint64_t n, void *stream) {
    if (n == 0) return B3G_OK;
    if (offsets == nullptr || lengths == nullptr || out == nullptr) return B3G_EINVAL;
    if (reinterpret_cast<uintptr_t>(base) % 16 != 0) return B3G_EALIGN;
    if (reinterpret_cast<uintptr_t>(keys) % 16 != 0) return B3G_EALIGN;  // read as 16-byte words
    for (uint64_t i = 0; i < n; ++i) {
        if (offsets[i] % 16 != 0) return B3G_EALIGN;
        if (lengths[i] > kMaxMessageBytes) return B3G_ETOOBIG;
        if (lengths[i] > 0 && base == nullptr) return B3G_EINVAL;
        if (offsets[i] + lengths[i] < offsets[i]) return B3G_EINVAL;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Equal lengths at evenly spaced offsets: the geometry is implied, no task table.
    const uint64_t stride = n > 1 ? offsets[1] - offsets[0] : 0;
    bool uniform = !uniform_batch_disabled();
    for (uint64_t i = 1; uniform && i < n; ++i)
        uniform = lengths[i] == lengths[0] && offsets[i] - offsets[i - 1] == stride;
    if (uniform)
        return hash_uniform(static_cast<const uint8_t *>(base) + offsets[0], stride, lengths[0], n, keys,
                            kIV, keys ? kKeyedHash : 0u, 0, kRoot, static_cast<uint8_t *>(out), s);

    // The task table is read by the device from host memory that later calls reuse (or
    // that is freed on return): a graph that recorded the upload would read another
    // call's table when replayed. Such a batch is refused under capture.
    // (A failed query means no capture: the calls below report what is wrong.)
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
        (void)hipGetLastError();
        cap = hipStreamCaptureStatusNone;
    }
    if (cap != hipStreamCaptureStatusNone) return B3G_EINVAL;

    uint64_t total_chunks = 0;
    for (uint64_t i = 0; i < n; ++i) total_chunks += chunks_of(lengths[i]);
    BatchPlan plan;
    int rc = plan_batch(lengths, n, kLeafLanes, choose_chunks_per_lane(total_chunks), kLevelLanes, &plan);
    if (rc != B3G_OK) return rc;

    // Scratch layout: message table, then per pass (segments, first-segment index, levels),
    // then one CV array per pass output. Everything but the CV arrays is built on the host
    // and copied with one transfer.
    const size_t off_bytes = align256(n * 8);
    size_t at = 0;
    const size_t msg_off_at = at;
    at += off_bytes;
    const size_t msg_len_at = at;
    at += off_bytes;
    struct PassLayout {
        size_t segs, first, levels, cv_out;
    };
    std::vector<PassLayout> lay(plan.passes.size());
    for (size_t p = 0; p < plan.passes.size(); ++p) {
        const PassPlan &pp = plan.passes[p];
        lay[p].segs = at;
        at += align256(pp.segs.size() * sizeof(Seg));
        lay[p].first = at;
        at += align256(pp.wg_first_seg.size() * sizeof(uint32_t));
        lay[p].levels = at;
        at += align256(pp.wg_levels.size());
    }
    // Fused first level pass (the leaf launch reduces it, last arrival of each level
    // segment): the table also maps each leaf output CV to its level segment, and the
    // level segments' tickets come from the scratch slot (zero, and left at zero).
    const bool fuse = fuse_batch_first_level(plan) && !use_lds_staging() &&
                      plan.passes[1].segs.size() <= kSlotTicketWords;
    size_t up_at = 0;
    if (fuse) {
        up_at = at;
        at += align256(plan.passes[1].up.size() * sizeof(uint32_t));
    }
    const size_t table_bytes = at;
    for (size_t p = 0; p < plan.passes.size(); ++p) {
        lay[p].cv_out = at;
        at += align256(plan.passes[p].out_cvs * 32);
    }
    StreamScratch scratch(s);
    rc = scratch.alloc(at);
    if (rc != B3G_OK) return rc;
    uint8_t *d = scratch.get();
    uint32_t *tickets = fuse ? scratch.zeroed_tickets(plan.passes[1].segs.size()) : nullptr;

    // the table image (the alignment padding between its parts is never read and left as
    // it is): in a pinned buffer, uploaded by a copy kernel, when one is free; else in
    // pageable memory, copied by the runtime
    TableStage stage;
    std::unique_ptr<uint8_t[]> pageable;
    uint8_t *img = stage.take(table_bytes);
    const bool pinned = img != nullptr;
    if (!pinned) {
        pageable.reset(new uint8_t[table_bytes]);
        img = pageable.get();
    }
    memcpy(img + msg_off_at, offsets, n * 8);
    memcpy(img + msg_len_at, lengths, n * 8);
    for (size_t p = 0; p < plan.passes.size(); ++p) {
        copy_bytes(img, lay[p].segs, plan.passes[p].segs);
        copy_bytes(img, lay[p].first, plan.passes[p].wg_first_seg);
        copy_bytes(img, lay[p].levels, plan.passes[p].wg_levels);
    }
    if (fuse) copy_bytes(img, up_at, plan.passes[1].up);
    if (pinned) {
        rc = stage.upload(d, table_bytes, s);
        if (rc != B3G_OK) return rc;
    } else if (hipMemcpyAsync(d, img, table_bytes, hipMemcpyHostToDevice, s) != hipSuccess) {
        return launched(hipErrorUnknown);
    }

    for (size_t p = 0; p < plan.passes.size(); ++p) {
        const PassPlan &pp = plan.passes[p];
        const auto *segs = reinterpret_cast<const Seg *>(d + lay[p].segs);
        const auto *first = reinterpret_cast<const uint32_t *>(d + lay[p].first);
        const auto *levels = reinterpret_cast<const uint8_t *>(d + lay[p].levels);
        auto *cv_out = reinterpret_cast<uint32_t *>(d + lay[p].cv_out);
        if (p == 0) {
            BatchLeafArgs a{static_cast<const uint8_t *>(base),
                            reinterpret_cast<const uint64_t *>(d + msg_off_at),
                            reinterpret_cast<const uint64_t *>(d + msg_len_at),
                            keys, first, levels, segs, cv_out, static_cast<uint8_t *>(out),
                            nullptr, nullptr, nullptr, nullptr};
            const bool fused = tickets != nullptr;
            if (fused) {
                a.up = reinterpret_cast<const uint32_t *>(d + up_at);
                a.lvl_segs = reinterpret_cast<const Seg *>(d + lay[1].segs);
                a.lvl_ctr = tickets;
                a.lvl_cv_out = reinterpret_cast<uint32_t *>(d + lay[1].cv_out);
            }
            rc = launched(launch_batch_leaf(a, pp.chunks_per_lane, use_lds_staging(), fused, pp.workgroups(), s));
            if (fused) ++p;  // the first level pass ran in the leaf launch
        } else {
            const auto *cv_in = reinterpret_cast<const uint32_t *>(d + lay[p - 1].cv_out);
            BatchLevelArgs a{cv_in, keys, first, levels, segs, cv_out, static_cast<uint8_t *>(out)};
            rc = launched(launch_batch_level(a, pp.workgroups(), s));
        }
        if (rc != B3G_OK) return rc;
    }
    return B3G_OK;
}

}  // namespace
}  // namespace b3g

extern "C" {

int blake3_gpu_hash(const void *dev_in, uint64_t len, void *dev_out32, void *stream) {
    return b3g::hash_single(dev_in, len, b3g::kIV, 0, dev_out32, stream);
}

int blake3_gpu_keyed_hash(const void *dev_in, uint64_t len, const uint32_t key[8], void *dev_out32,
                          void *stream) {
    if (key == nullptr) return B3G_EINVAL;
    return b3g::hash_single(dev_in, len, key, b3g::kKeyedHash, dev_out32, stream);
}

int blake3_gpu_keyed_hash_noalloc(const void *dev_in, uint64_t len, const uint32_t key[8], void *dev_out32,
                                  void *stream) {
    return b3g::hash_single(dev_in, len, key ? key : b3g::kIV, key ? b3g::kKeyedHash : 0u, dev_out32, stream,
                            true);
}

int blake3_gpu_keyed_hash_batch(const void *dev_base, const uint64_t *host_offsets,
                                const uint64_t *host_lengths, const uint32_t *dev_keys, void *dev_out,
                                uint64_t n, void *stream) {
    return b3g::hash_batch(dev_base, host_offsets, host_lengths, dev_keys, dev_out, n, stream);
}

int blake3_gpu_subtree_cv(const void *dev_in, uint64_t len, uint64_t chunk_base, const uint32_t key[8],
                          void *dev_out32, void *stream) {
    return b3g::subtree_cv(dev_in, len, chunk_base, key, dev_out32, stream);
}

int blake3_gpu_hash_xof(const void *dev_in, uint64_t len, const uint32_t key[8], void *dev_out, uint64_t out_len,
                        void *stream) {
    return b3g::hash_xof(dev_in, len, key, 0, dev_out, out_len, stream);
}

int blake3_gpu_hash_xof_at(const void *dev_in, uint64_t len, const uint32_t key[8], uint64_t out_offset,
                           void *dev_out, uint64_t out_len, void *stream) {
    return b3g::hash_xof(dev_in, len, key, out_offset, dev_out, out_len, stream);
}

int blake3_gpu_group_cvs(const void *dev_in, uint64_t len, uint64_t chunk_base, const uint32_t key[8],
                         uint32_t group_chunks, void *dev_cvs, void *stream) {
    return b3g::group_cvs(dev_in, len, chunk_base, key, group_chunks, dev_cvs, stream);
}

uint32_t blake3_gpu_leaf_group_chunks(uint64_t len) {
    const uint64_t c = b3g::chunks_of(len);
    if (c <= b3g::quad_leaf_max_chunks()) return b3g::kQuadLeafChunks;
    if (const uint32_t ks = b3g::split_tail_chunks_per_lane(c)) return b3g::kLeafLanes * ks;
    return b3g::kLeafLanes * b3g::choose_single_chunks_per_lane(c);
}

const char *blake3_gpu_strerror(int status) {
    switch (status) {
        case B3G_OK: return "success";
        case B3G_EINVAL: return "invalid argument (NULL pointer or offset overflow)";
        case B3G_EALIGN: return "a device pointer or batch offset is not 16-byte aligned";
        case B3G_ENOMEM: return "scratch allocation failed";
        case B3G_EHIP: return "HIP runtime call or kernel launch failed";
        case B3G_ETOOBIG: return "request exceeds the supported size";
        case B3G_ESCRATCH:
            return "the input needs more scratch than the fixed array of the no-allocation entry point holds";
        default: return "unknown status";
    }
}

int blake3_gpu_version(void) { return b3g::kAbiVersion; }

int blake3_gpu_debug_reload_env(void) {
    b3g::reload_options();
    return B3G_OK;
}

int64_t blake3_gpu_debug_plan_batch(const uint64_t *host_lengths, uint64_t n, uint64_t *out,
                                    uint64_t out_words) {
    if (n > 0 && host_lengths == nullptr) return B3G_EINVAL;
    uint64_t total_chunks = 0;
    for (uint64_t i = 0; i < n; ++i) total_chunks += b3g::chunks_of(host_lengths[i]);
    b3g::BatchPlan plan;
    const int rc = b3g::plan_batch(host_lengths, n, b3g::kLeafLanes, b3g::choose_chunks_per_lane(total_chunks),
                                   b3g::kLevelLanes, &plan);
    if (rc != B3G_OK) return rc;
    std::vector<uint64_t> w;
    w.push_back(plan.passes.size());
    for (const b3g::PassPlan &p : plan.passes) {
        w.push_back(p.lanes);
        w.push_back(p.chunks_per_lane);
        w.push_back(p.workgroups());
        w.push_back(p.segs.size());
        w.push_back(p.in_cvs);
        w.push_back(p.out_cvs);
        for (uint32_t f : p.wg_first_seg) w.push_back(f);
        for (uint8_t l : p.wg_levels) w.push_back(l);
        for (const b3g::Seg &g : p.segs) {
            w.push_back(g.msg);
            w.push_back(g.first);
            w.push_back(g.dst);
            w.push_back(g.info);
        }
    }
    if (out != nullptr && out_words >= w.size()) memcpy(out, w.data(), w.size() * sizeof(uint64_t));
    return static_cast<int64_t>(w.size());
}

}  // extern "C"
