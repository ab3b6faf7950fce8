// ddh_internal.h - plan state and device descriptors shared by the library's
// translation units (map builder, exchange kernels, C ABI). Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/ddh.h"

namespace ddh {

// A named host range (an entry point, a phase of the map build), seen by
// rocprofv3 --marker-trace; a no-op without a profiler.
struct Range {
    explicit Range(const char* name) { roctxRangePushA(name); }
    ~Range() { roctxRangePop(); }
    Range(const Range&) = delete;
    Range& operator=(const Range&) = delete;
};

// Work-group size of the per-pulse and helper kernels (four 64-wide
// wavefronts); the fused launch picks 256 or 1024.
constexpr int kBlock = 256;

// Control words, each on its own 128-byte line (index in uint32 units).
enum CtrlWord : int {
    kCtrlPassX = 0,    // fused coordinate passes completed (counter targets)
    kCtrlPassF = 32,   // fused force passes completed
    kCtrlEpochX = 64,  // coordinate passes completed in any mode (flag values)
    kCtrlEpochF = 80,  // force passes completed in any mode
    kCtrlTicket = 96,  // next dynamic work ticket of the running fused launch
    kCtrlDone = 128,   // work-groups that left the running fused launch
    kCtrlPulseDone = 160,  // blocks that left the running per-pulse launch
                           // that publishes its own flags at exit
    kCtrlError = 192,  // first device-side error code (0 = none)
    kCtrlWords = 224
};

// One work chunk of one (sender S, pulse p) map: 64 bytes, read with one
// scalar load. A map with c chunks gives chunk k the k-th of c slices of its
// independent head (entries below the sender's home count) and, for the
// coordinate pass, the k-th slice of its dependent tail (forwarded records),
// so the dependent work of a map is spread over c work-groups.
struct DChunk {
    int32_t hb, he;      // independent entries [hb, he) of the map
    int32_t tb, te;      // coordinates: dependent entries [tb, te); forces: empty
    uint32_t wait_a;     // coords: pulses q whose region at S the tail reads
                         // forces: later pulses q whose (S, q) map must be done
    uint32_t wait_b;     // forces: later pulses q whose (R, q) map must be done
    int32_t src_base;    // first slot of sender S
    int32_t dst_base;    // first slot of the region at receiver R
    int32_t map_off;     // first entry of the (S, p) map in the map array
    int32_t flags;       // bits 0-7: pulse dimension d; kChunkShift: component d
                         // gets + shift; kChunkRelease: later chunks of the same
                         // launch read what this chunk writes (publish with a
                         // release fence)
    int32_t unused;
    float shift;         // L_d
    int32_t S, R;
    int32_t ctr;         // counter this chunk advances: coords R*P+p, forces S*P+p
    int32_t p;
};
constexpr int32_t kChunkShift = 1 << 8;
constexpr int32_t kChunkRelease = 1 << 9;
static_assert(sizeof(DChunk) == 64, "DChunk layout");

// Kernel arguments of one fused launch (passed by value). Tickets
// [0, nx) are coordinate chunks, [nx, nx + nf) force chunks.
struct XArgs {
    float* x;
    float* f;
    const void* maps;        // map entries in the kernel's index type (int32
                             // or uint16)
    const DChunk* xchunks;
    const DChunk* fchunks;
    int32_t nx, nf;
    uint32_t* ctrl;
    uint32_t* xcnt;          // [R*P+p] chunks that filled region p of R, all passes
    uint32_t* fcnt;          // [S*P+p] chunks of item (S, p) that added, all passes
    const uint32_t* xneed;   // [R*P+p] chunks per pass behind xcnt
    const uint32_t* fneed;   // [S*P+p] chunks per pass behind fcnt
    int32_t P;
    int32_t static_first;    // 1: work-group b starts with ticket b
    int32_t force_timeout;   // waits target a value nobody writes
    uint32_t spin_limit;
    uint64_t* trace;         // optional event log (null: off)
    uint32_t* flags;         // per-pulse completion flags, published at exit
};

// Event log: work-group b writes record k at trace[2 * (b * kTraceRecords + k)]
// as (code << 32 | info, wall-clock ticks of the 100 MHz constant counter).
constexpr int kTraceRecords = 64;
enum TraceCode : uint32_t {
    kTrStart = 1,    // info: grid size
    kTrClaim = 2,    // info: ticket
    kTrHead = 3,     // info: entries of the independent part done
    kTrWaited = 4,   // info: wait masks
    kTrChunk = 5,    // info: entries of the chunk done
    kTrPublish = 6,  // info: counter advanced
    kTrExit = 7
};

struct Geometry {
    int n[3] = {1, 1, 1};
    float L[3] = {0, 0, 0};
    float rc = 0, cell = 0, inv_c = 0;
    std::vector<float> b[3];      // boundaries, n[d] + 1 per dimension
    std::vector<int> ncell[3];    // sort cells across domain index i of d
    int ndom = 1;
    int P = 0;
    int pdim[DDH_MAX_PULSES] = {0};
    int pk[DDH_MAX_PULSES] = {0};
    void coords(int D, int c[3]) const {
        c[0] = D % n[0];
        c[1] = (D / n[0]) % n[1];
        c[2] = D / (n[0] * n[1]);
    }
    int index(const int c[3]) const { return c[0] + n[0] * (c[1] + n[1] * c[2]); }
};

// The chunks of one execution mode: coordinate chunks in pulse order, force
// chunks in decreasing pulse order, each pulse's chunks contiguous.
struct WorkTable {
    int chunk = 0;                  // entries per chunk
    bool wave = false;              // fused: built for wavefront workers
    bool heads_first = false;       // fused: every map's head in chunks of its
                                    // own, all heads before any tail
    std::vector<int32_t> nchunks;   // [S * P + p] chunks of the map
    std::vector<DChunk> xch, fch;   // host copies (fused table only; the
                                    // per-pulse tables are made on the device)
    int nx = 0, nf = 0;             // coordinate and force chunks
    std::vector<int32_t> xpulse_begin, fpulse_begin;  // per pulse ranges (+1)
    DChunk* d_xch = nullptr;        // device copies
    DChunk* d_fch = nullptr;
    // per-pulse launches: the map entries of coordinate chunk k at
    // [k * chunk, k * chunk + size) (then zeros), so a block finds its
    // entries from its chunk index alone and loads them while its
    // descriptor is still in flight; kPadTail zero entries follow the last
    // chunk. Force chunks use the slots of the coordinate chunk of the same
    // map slice. 16-bit when the maps have a 16-bit copy; 32-bit when they
    // have none or the build ran with the 16-bit maps off (else null).
    int32_t* d_pad = nullptr;
    uint16_t* d_pad16 = nullptr;
};
constexpr int kSmallChunk = 256;   // per-pulse chunk where launches are latency-bound
constexpr int kPadTail = 4096;      // >= entries per round of any block

// The passes an exchange call runs.
enum Op : int { kOpCoords = 1, kOpForces = 2, kOpStep = 3 };

struct Plan {
    int device = 0;
    int n_cu = 256;
    Geometry g;
    bool built = false;
    int32_t n_atoms = 0;
    int64_t n_slots = 0;
    int64_t n_halo = 0;
    int32_t mode = DDH_MODE_AUTO;   // as requested (ddh_set_mode)
    // FUSED or PULSE (plus the GRAPH bit): AUTO resolved against the layout
    // and against how the call's launches will run (replayed from a graph:
    // captured by the caller or DDH_MODE_GRAPH; else enqueued eagerly)
    int32_t effective_mode(bool captured) const
    {
        const int32_t base = mode & ~DDH_MODE_GRAPH;
        const bool replayed = captured || (mode & DDH_MODE_GRAPH);
        const int32_t m = base != DDH_MODE_AUTO ? base
                          : (!replayed && n_halo <= DDH_AUTO_FUSED_MAX) ? DDH_MODE_FUSED
                                                                        : DDH_MODE_PULSE;
        return m | (mode & DDH_MODE_GRAPH);
    }
    // whether some call under the current mode can run the fused launch:
    // FUSED, or AUTO on eager calls over a small layout
    bool may_fuse() const
    {
        const int32_t base = mode & ~DDH_MODE_GRAPH;
        return base == DDH_MODE_FUSED ||
               (base == DDH_MODE_AUTO && !(mode & DDH_MODE_GRAPH) && n_halo <= DDH_AUTO_FUSED_MAX);
    }

    // tuning
    int chunk_req = 0;
    int grid_req = 0;
    int block_req = 0;          // fused work-group width: 0 automatic, 256 or 1024
    int static_first = 0;       // fused: first tickets unclaimed (exclusive GPU)
    int flags = 1;              // publish the per-pulse completion flags
    uint32_t spin_limit = 1u << 20;
    int force_timeout = 0;
    int refined_waits = 1;
    int narrow_maps = 1;        // use the 16-bit copy of the maps when there is one
    int wave_chunks = 0;        // fused: wavefront workers on contiguous slices
                                // (takes effect at the next build)
    int home_sort = 0;          // home-atom sort of the build: 0 automatic,
                                // 1 counting sort, 2 partition sort
    int heads_first = 0;        // fused: heads-first ticket order (next build)
    int exit_publish = 0;       // per-pulse mode: 0 automatic, 1 the last
                                // launch publishes its flags at exit, 2 a
                                // one-wave launch after it does
    int lds_stage = 0;          // per-pulse and fused: coordinate stores staged through LDS
                                // (1 gathered in registers, 2 by LDS loads)
    int pad_maps = 0;           // per-pulse mode: 0 automatic, 1 blocks read
                                // the chunk-aligned map copy (loads issued
                                // before the descriptor arrives), 2 the maps
                                // themselves, after the descriptor
    uint64_t* trace = nullptr;  // caller-owned device buffer (DDH_TUNE_TRACE)

    // host copies of the layout
    std::vector<int64_t> base;     // per domain
    std::vector<int32_t> nhome, ntotal;
    std::vector<int32_t> send, split, recv, roff, shift;  // [S * P + p]
    std::vector<int64_t> map_off;  // [S * P + p]
    WorkTable fused;               // fused launch: waits and release flags set
    WorkTable pulse;               // per-pulse launches of step calls (both
                                   // passes per launch): no waits
    WorkTable pulse1;              // per-pulse launches of single-pass calls
                                   // (a launch carries half the work: smaller
                                   // chunks); unused (chunk 0) when it would
                                   // equal the step table
    const WorkTable& pulse_table(int op) const
    {
        return (op == kOpStep || pulse1.chunk == 0) ? pulse : pulse1;
    }

    // device state
    int32_t* d_maps = nullptr;     // all maps, pulse-major
    uint16_t* d_maps16 = nullptr;  // the same entries as 16 bits, when every
                                   // domain has at most 65536 slots (else null)
    int32_t* d_slot_gid = nullptr; // global id per slot
    int32_t* d_home_gid = nullptr; // home atoms in slot order, all domains
    int32_t* d_home_slot = nullptr;
    uint8_t* d_rid = nullptr;      // per slot: the pulse that delivered it (0xff: home)
    bool fused_ready = false;      // the fused launch's table and counter targets
                                   // are made (at the build, or at the first
                                   // switch to a mode that may run that launch)
    bool fused_refined = true;     // refined waits, as set at the build
    uint32_t* d_ctrl = nullptr;    // control words, then the arrays below
    uint32_t* d_xcnt = nullptr;
    uint32_t* d_fcnt = nullptr;
    uint32_t* d_xneed = nullptr;
    uint32_t* d_fneed = nullptr;
    uint32_t* d_pflag = nullptr;   // per-pulse completion flags: [p] coordinates,
                                   // [DDH_MAX_PULSES + p] forces (epoch values)
    float* d_stage = nullptr;      // staging buffer of DDH_MODE_STAGED (first use)
    std::vector<void*> owned;      // allocations made after the build (staging buffer)
    std::vector<std::pair<void*, size_t>> kept;     // built state, reused by later builds
    size_t kept_next = 0;          // next slot of kept during a build
    std::vector<std::pair<void*, size_t>> scratch;  // build scratch, kept between builds
    std::vector<std::pair<void*, size_t>> pinned;   // pinned host staging of the build's
                                                    // uploads, kept between builds
    // per pulse: the selection's output (map entries, received ids and
    // positions; 20 bytes per entry) and its room in entries, sized from
    // earlier builds with a quarter to spare, so a pulse's write is enqueued
    // before its counts reach the host
    std::vector<std::pair<void*, size_t>> selbuf;
    hipEvent_t counts_ready = nullptr;  // the build's count read-back has landed
    bool build_failed = false;     // the last build returned an error midway

    // graph replay cache: (op, x, f, mode) -> executable graph
    hipStream_t capture_stream = nullptr;
    std::map<std::tuple<int, void*, void*, int>, hipGraphExec_t> graphs;
};

// Work item of work-group b of n, dealt so that neighbouring items share an
// XCD: the hardware deals work-groups to the eight XCDs in turn (work-group b
// runs on XCD b % 8), and XCD k takes the k-th contiguous eighth of the
// items instead, so items whose data share cache lines go through one L2. A
// permutation of [0, n): results do not depend on it.
__device__ __forceinline__ int xcd_tile(int b, int n)
{
    const int per = n / 8, rem = n % 8;  // XCD k takes per + (k < rem) items
    const int k = b % 8;
    return k * per + (k < rem ? k : rem) + b / 8;
}

// Work item of work-group b of n when groups of G neighbouring items should
// share an XCD but every XCD should still see items from the whole range:
// the XCDs take groups of G items in turn (work-groups in whole rounds of
// 8 * G; the rest keep their own index). A permutation of [0, n).
template <int G>
__device__ __forceinline__ int xcd_group(int b, int n)
{
    constexpr int span = 8 * G;
    if (b >= n / span * span)
        return b;
    const int i = b / 8;  // the i-th work-group of XCD b % 8
    return i / G * span + b % 8 * G + i % G;
}

// error reporting (thread-local text)
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);

#define DDH_HIP(call)                                          \
    do {                                                       \
        hipError_t _e = (call);                                \
        if (_e != hipSuccess) return ddh::hip_fail(_e, #call); \
    } while (0)

// map builder (ddh_build.hip)
int build_maps(Plan* plan, const float* xg, int32_t n_atoms, hipStream_t stream);
void free_built(Plan* plan);
// the fused launch's table, wait masks and counter targets for the current
// build, on the plan's own stream (waits for it)
int prepare_fused(Plan* plan);
void free_scratch(Plan* plan);

// exchange launches (ddh_exchange.hip)
int enqueue_exchange(Plan* plan, int op, float* x, float* f, hipStream_t stream);
int enqueue_gather_home(Plan* plan, const float* xg, float* x, hipStream_t stream);
int enqueue_wait_flag(Plan* plan, int idx, uint32_t epoch, hipStream_t stream);
// the host-orchestrated exchange with its staging in the library's static
// device array (no allocation); at most kStaticStageBytes of staging
constexpr size_t kStaticStageBytes = (size_t)DDH_STATIC_STAGE_BYTES;
int enqueue_staged_static(Plan* plan, int op, float* x, float* f, hipStream_t stream);

}  // namespace ddh
