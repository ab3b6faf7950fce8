// ddh_exchange.hip - coordinate and force passes of the staged halo exchange
// on gfx950, plus the home-slot gather.
//
// Source ("the guide"): NVIDIA technical blog "A Practical Guide to
// GPU-Initiated Communication for Molecular Dynamics at Scale".
//
// Every domain is a slice of one device array, so the guide's direct-store
// path ("Optimizing for efficient transfers across NVIDIA NVLink-connected
// GPUs") is the main path: a sender gathers its map entries and stores them
// straight into the receiver's slots; nothing is staged and nothing is "put".
// The work of a pass is cut into chunks (DChunk: a slice of one (sender,
// pulse) map). Three ways to run them:
//
//  - Per-pulse launches (DDH_MODE_PULSE; the guide's stream-ordered design of
//    "Replacing host-side communication with NVSHMEM"): one launch per pulse,
//    its blocks loop over the pulse's chunks; the stream orders the pulses,
//    so no kernel waits, counts or fences. A step call runs coordinate pulse
//    q and force pulse P-1-q in the same launch. A one-wave launch afterwards
//    publishes per-pulse flags. The default whenever the calls are replayed
//    from a graph: on MI355X a kernel boundary inside a graph costs less than
//    a dependency carried across XCDs inside a kernel.
//
//  - One fused launch per call (DDH_MODE_FUSED; "Enabling parallelism across
//    pulses through kernel fusion", "Dependency-aware packing", "Force halo
//    exchange: Reversing the dependency chain"): work-groups claim chunks in
//    ticket order (a chunk only ever waits on chunks claimed before it, so
//    the launch cannot deadlock whatever the grid size or whatever else runs
//    on the GPU). A coordinate chunk packs its independent slice, waits until
//    the regions its dependent slice reads are complete, then packs that
//    slice; a force chunk waits until the later pulses that add into the same
//    slots of S, or into the slots of R's region it reads, are done, so each
//    slot receives its adds in decreasing pulse order and matches the
//    sequential reverse pass bit for bit. The single-launch form, and the
//    default for eager calls on small passes, where the host's cost per
//    launch dominates. With DDH_TUNE_WAVE_CHUNKS the same launch runs
//    wave_kernel, in which every wavefront is an independent worker on
//    contiguous map slices ("NVLink path: TMA-based direct stores").
//
//  - The host-orchestrated baseline (DDH_MODE_STAGED; "From MPI baseline to
//    optimized GPU-native halo exchange"): pack into a staging buffer, host
//    wait, one copy per sender, host wait; forces the reverse.
//
// Completion in the fused launch ("Dependency-aware packing", hierarchical
// release): every wave of a chunk's work-group waits for its own stores, then
// thread 0 issues one agent-scope release fence and a relaxed increment of
// the map's counter. The counters only grow, one step per chunk and pass, so
// a waiter polls until a counter reaches pass * chunks-per-pass and then
// acquires: every increment continues the release sequence of the earlier
// ones, and no counter or flag is ever reset. All eight XCDs form one agent,
// so agent scope plays the role the guide gives to system scope. On MI355X
// each agent-scope fence and each same-address atomic is serialized
// device-wide (tens of ns), which is why chunks are large and a chunk issues
// one fence, not one per entry.
//
// Every wait is bounded by a spin limit; on expiry it records DDH_ETIMEOUT in
// the control block and the work-group carries on, so every launch drains.
#pragma clang fp contract(off)

#include <mutex>

#include "ddh_internal.h"

namespace ddh {

namespace {

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void add_relaxed(uint32_t* p, uint32_t v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Event log of thread 0 (see kTraceRecords); a no-op without a buffer.
__device__ __forceinline__ void trace_rec(const XArgs& a, int& n, uint32_t code, uint32_t info)
{
    if (a.trace && n < kTraceRecords) {
        uint64_t* r = a.trace + 2ull * ((uint64_t)blockIdx.x * kTraceRecords + n);
        r[0] = ((uint64_t)code << 32) | info;
        r[1] = wall_clock64();
        n++;
    }
}

// Index of the n-th set bit of m (n < popcount(m)).
__device__ __forceinline__ int nth_bit(uint32_t m, int n)
{
    for (; n > 0; n--)
        m &= m - 1;
    return __builtin_ctz(m);
}

// Wait until every vector memory operation this wave issued has completed
// (s_waitcnt vmcnt 0; expcnt and lgkmcnt left at their maxima, so no wait on
// them). Needed wherever one wave's fence or barrier stands for the whole
// work-group: an agent-scope fence waits only for the wave that executes it,
// and __syncthreads() emits no vmcnt wait on gfx950 (a workgroup-scope
// release needs none, since the waves share the CU).
__device__ __forceinline__ void wait_vm_idle()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Wave 0 waits for every counter a chunk needs at once: lane l polls the
// l-th of (the counters of the pulses in mask_a at row_a; those in mask_b at
// row_b), so one round trip checks them all. The loop exit is a wave-wide
// vote. Ends with an acquire fence.
__device__ void wave_wait(const XArgs& a, const uint32_t* cnt, const uint32_t* need, uint32_t pass,
                          uint32_t mask_a, int row_a, uint32_t mask_b, int row_b, uint32_t bump)
{
    const int l = (int)(threadIdx.x & 63);
    const uint32_t* ptr = nullptr;
    uint32_t target = 0;
    const int na = __builtin_popcount(mask_a);
    if (l < na) {
        const int r = row_a + nth_bit(mask_a, l);
        ptr = cnt + r;
        target = pass * need[r] + bump;
    } else if (l - na < __builtin_popcount(mask_b)) {
        const int r = row_b + nth_bit(mask_b, l - na);
        ptr = cnt + r;
        target = pass * need[r] + bump;
    }
    uint32_t n = 0;
    for (;;) {
        const bool ok = !ptr || (int32_t)(ld_relaxed(ptr) - target) >= 0;
        if (__all(ok))
            break;
        if (++n >= a.spin_limit) {
            if (l == 0) {
                uint32_t zero = 0;
                __hip_atomic_compare_exchange_strong(a.ctrl + kCtrlError, &zero,
                                                     (uint32_t)DDH_ETIMEOUT, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // the invalidation has completed before the barrier that lets the
    // work-group's other waves read
    wait_vm_idle();
}

// A chunk descriptor through the scalar cache: the tables are read-only
// for the whole launch and the index is uniform across the block, so one
// s_load fetches all 64 bytes without occupying the vector memory counter.
typedef const __attribute__((address_space(4))) uint32_t* ConstWordPtr;

__device__ __forceinline__ DChunk load_chunk(const DChunk* table, int k)
{
    const ConstWordPtr w = (ConstWordPtr)(table + k);
    uint32_t words[sizeof(DChunk) / 4];
#pragma unroll
    for (int i = 0; i < (int)(sizeof(DChunk) / 4); i++)
        words[i] = w[i];
    DChunk c;
    __builtin_memcpy(&c, words, sizeof(DChunk));
    return c;
}

// Map entries of one round: entry i0 + e * B + tid for e < E. B threads
// share a round: a whole work-group (B = its width, tid = threadIdx.x) or one
// wavefront (B = 64, tid = its lane). I is the stored index type: int32, or
// uint16 when every domain has at most 65536 slots (half the bytes for the
// same entries).
template <int E, int B, typename I>
__device__ __forceinline__ void load_map(const I* map, int i0, int end, int (&j)[E])
{
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int i = i0 + e * B + (int)threadIdx.x % B;
        j[e] = i < end ? (int)map[i] : -1;
    }
}

// The two halves of one round, for a caller that issues other loads between
// them (the per-pulse kernel's prefetch of its next chunk): the reads of the
// round into registers, then the adds, shifts and stores.
// The reads are unconditional, so a lane's E gathers issue back to back with
// no branch between them: an entry past the chunk's end (j < 0) reads the
// sender's first slot instead, which exists whenever the chunk has entries,
// and its value is never stored.
template <int E, int B>
__device__ __forceinline__ void coords_gather(const float* src, const int (&j)[E], float (&v)[E][3])
{
#pragma unroll
    for (int e = 0; e < E; e++) {
        const float* s = src + 3ll * (j[e] < 0 ? 0 : j[e]);
        v[e][0] = s[0];
        v[e][1] = s[1];
        v[e][2] = s[2];
    }
}

template <int E, int B>
__device__ __forceinline__ void coords_put(float* dst, const DChunk& c, int i0, int end,
                                           float (&v)[E][3])
{
    // + L on the pulse's component at a shifting sender, as a select (the
    // other components are left untouched, not added 0, so a -0.0 stays)
    const bool shift = (c.flags & kChunkShift) != 0;
    const int dd = c.flags & 0xff;
#pragma unroll
    for (int e = 0; e < E; e++)
#pragma unroll
        for (int k = 0; k < 3; k++)
            v[e][k] = (shift && dd == k) ? v[e][k] + c.shift : v[e][k];
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int i = i0 + e * B + (int)threadIdx.x % B;
        if (i < end) {
            float* d = dst + 3ll * i;
            __builtin_nontemporal_store(v[e][0], d);
            __builtin_nontemporal_store(v[e][1], d + 1);
            __builtin_nontemporal_store(v[e][2], d + 2);
        }
    }
}

// LDS-staged form of coords_put: per round, each wavefront's 64 records
// form one contiguous run of the destination (768 bytes). The wavefront
// writes the runs of all its rounds into its LDS tile, each at the run's
// 16-byte alignment, then stores every run from the tile in 16-byte groups:
// one aligned dwordx4 per lane for the groups the run fills, and one dword
// store instruction for the at most six dwords of the two groups the run
// starts and ends inside (lanes 56-61, which no group uses: a run touches at
// most 49 groups). tile holds E * kStageTile floats per wavefront, 16-byte
// aligned.
constexpr int kStageTile = 196;  // 192 dwords of a run + up to 3 of alignment, rounded to 16 B
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int E, int B>
__device__ __forceinline__ void coords_put_lds(float* dst, const DChunk& c, int i0, int end,
                                               float (&v)[E][3], float* tile)
{
    const bool shift = (c.flags & kChunkShift) != 0;
    const int dd = c.flags & 0xff;
#pragma unroll
    for (int e = 0; e < E; e++)
#pragma unroll
        for (int k = 0; k < 3; k++)
            v[e][k] = (shift && dd == k) ? v[e][k] + c.shift : v[e][k];
    const int lane = (int)threadIdx.x & 63;
    const int w = ((int)threadIdx.x % B) >> 6;
    const int seg0 = i0 + w * 64;  // round e's run starts at entry seg0 + e * B
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int seg = seg0 + e * B;
        const int a = (int)(((uintptr_t)(dst + 3ll * seg) >> 2) & 3);  // dwords before it in its group
        float* t = tile + e * kStageTile + a + 3 * lane;
        if (seg + lane < end) {
            t[0] = v[e][0];
            t[1] = v[e][1];
            t[2] = v[e][2];
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int seg = seg0 + e * B;  // wavefront-uniform
        if (seg >= end)
            break;
        const int nd = 3 * min(64, end - seg);  // the run's dwords
        float* run = dst + 3ll * seg;
        const int a = (int)(((uintptr_t)run >> 2) & 3);
        float* base = run - a;  // 16-byte aligned
        const float* tl = tile + e * kStageTile;
        const int ng = (a + nd + 3) >> 2;  // 16-byte groups the run touches
        const bool head = a > 0 || nd < 4;          // group 0 is partial
        const bool tail = ng > 1 && ((a + nd) & 3);  // group ng - 1 is partial (and not group 0)
        if (lane < ng && !(lane == 0 && head) && !(lane == ng - 1 && tail)) {
            const float4v q = *reinterpret_cast<const float4v*>(tl + 4 * lane);
            __builtin_nontemporal_store(q, reinterpret_cast<float4v*>(base + 4 * lane));
        }
        // the partial groups' dwords, one lane each
        const int hn = head ? min(4, a + nd) - a : 0;
        const int tn = tail ? (a + nd) - 4 * (ng - 1) : 0;
        const int p = lane - 56;
        if (p >= 0 && p < hn + tn) {
            const int d = p < hn ? a + p : 4 * (ng - 1) + (p - hn);
            __builtin_nontemporal_store(tl[d], base + d);
        }
    }
    // the tile's reads are issued before a later round's writes
    wave_lds_sync();
}

// The same staging with the gathers done by the LDS's own loads
// (global_load_lds_dwordx3): each lane's 12-byte record goes from HBM into
// the wavefront's LDS tile without passing through registers. The load
// writes lane L's record at 16 L bytes of the round's tile (a 16-byte lane
// stride, the fourth dword untouched), so the stores read every dword of a
// 16-byte group from its record's place: dword r of a run is component r % 3
// of record r / 3, at tile float 4 (r / 3) + r % 3. Unconditional as in
// coords_gather (an entry past the end reads the sender's first slot). tile
// holds E * kDmaTile floats per wavefront.
constexpr int kDmaTile = 256;  // 64 lanes x 16 bytes
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

template <int E>
__device__ __forceinline__ void coords_dma_issue(const float* src, const int (&j)[E], float* tile)
{
#pragma unroll
    for (int e = 0; e < E; e++) {
        const float* s = src + 3ll * (j[e] < 0 ? 0 : j[e]);
        __builtin_amdgcn_global_load_lds((global_void*)s, (lds_void*)(tile + e * kDmaTile), 12, 0,
                                         0);
    }
}

template <int E, int B>
__device__ __forceinline__ void coords_dma_put(float* dst, const DChunk& c, int i0, int end,
                                               const float* tile)
{
    // vmcnt(0): every LDS load of the wavefront has landed (later loads
    // of the next chunk's maps are waited for too)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    wave_lds_sync();
    const bool shift = (c.flags & kChunkShift) != 0;
    const int dd = c.flags & 0xff;
    const int lane = (int)threadIdx.x & 63;
    const int w = ((int)threadIdx.x % B) >> 6;
    const int seg0 = i0 + w * 64;
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int seg = seg0 + e * B;  // wavefront-uniform
        if (seg >= end)
            break;
        const int nd = 3 * min(64, end - seg);
        float* run = dst + 3ll * seg;
        const int a = (int)(((uintptr_t)run >> 2) & 3);
        float* base = run - a;
        const float* tl = tile + e * kDmaTile;
        // dword d of the aligned groups (run dword d - a), shifted on the
        // pulse's component at a shifting sender
        auto rd = [&](int d) {
            const int r = d - a;
            const int rec = r / 3, k = r - 3 * rec;
            const float v = tl[4 * rec + k];
            return (shift && k == dd) ? v + c.shift : v;
        };
        const int ng = (a + nd + 3) >> 2;
        const bool head = a > 0 || nd < 4;
        const bool tail = ng > 1 && ((a + nd) & 3);
        if (lane < ng && !(lane == 0 && head) && !(lane == ng - 1 && tail)) {
            const int d = 4 * lane;
            const float4v q = {rd(d), rd(d + 1), rd(d + 2), rd(d + 3)};
            __builtin_nontemporal_store(q, reinterpret_cast<float4v*>(base + d));
        }
        const int hn = head ? min(4, a + nd) - a : 0;
        const int tn = tail ? (a + nd) - 4 * (ng - 1) : 0;
        const int p = lane - 56;
        if (p >= 0 && p < hn + tn) {
            const int d = p < hn ? a + p : 4 * (ng - 1) + (p - hn);
            __builtin_nontemporal_store(rd(d), base + d);
        }
    }
    // the tile's reads are issued before a later round's loads land
    wave_lds_sync();
}

// Unconditional as in coords_gather: an entry past the chunk's end reads the
// chunk's first region record and the sender's first slot.
template <int E, int B>
__device__ __forceinline__ void forces_gather(const float* from, const float* tgt, int i0,
                                              const int (&j)[E], float (&sv)[E][3],
                                              float (&tv)[E][3])
{
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int i = j[e] < 0 ? i0 : i0 + e * B + (int)threadIdx.x % B;
        const float* r = from + 3ll * i;
        sv[e][0] = r[0];
        sv[e][1] = r[1];
        sv[e][2] = r[2];
        const float* q = tgt + 3ll * (j[e] < 0 ? 0 : j[e]);
        tv[e][0] = q[0];
        tv[e][1] = q[1];
        tv[e][2] = q[2];
    }
}

template <int E, int B>
__device__ __forceinline__ void forces_put(float* tgt, const int (&j)[E], const float (&sv)[E][3],
                                           const float (&tv)[E][3])
{
#pragma unroll
    for (int e = 0; e < E; e++) {
        if (j[e] >= 0) {
            float* q = tgt + 3ll * j[e];
            __builtin_nontemporal_store(tv[e][0] + sv[e][0], q);
            __builtin_nontemporal_store(tv[e][1] + sv[e][1], q + 1);
            __builtin_nontemporal_store(tv[e][2] + sv[e][2], q + 2);
        }
    }
}

// One round of a range: x[dst + i] = x[src + map[i]] (+ L on the pulse's
// component) for the round's entries; all gathers are issued before any
// store. Stores are non-temporal: a region is written once per pass and not
// re-read by the writing work-group.
// STG 1: the stores are staged as in coords_put_lds; 2: the gathers are
// LDS loads as in coords_dma_put (tile: the wavefront's LDS tile).
template <int E, int B, int STG = 0>
__device__ __forceinline__ void coords_round(const float* src, float* dst, const DChunk& c, int i0,
                                             int end, const int (&j)[E], float* tile = nullptr)
{
    if constexpr (STG == 2) {
        coords_dma_issue<E>(src, j, tile);
        coords_dma_put<E, B>(dst, c, i0, end, tile);
    } else {
        float v[E][3];
        coords_gather<E, B>(src, j, v);
        if constexpr (STG == 1)
            coords_put_lds<E, B>(dst, c, i0, end, v, tile);
        else
            coords_put<E, B>(dst, c, i0, end, v);
    }
}

// Forces, one round: f[src + map[i]] += f[dst + i] (the receiver's region
// back into the sender's slots).
template <int E, int B>
__device__ __forceinline__ void forces_round(const float* from, float* tgt, int i0, int end,
                                             const int (&j)[E])
{
    float sv[E][3], tv[E][3];
    forces_gather<E, B>(from, tgt, i0, j, sv, tv);
    forces_put<E, B>(tgt, j, sv, tv);
}

// Entries [begin, end) of a chunk's map (map: the chunk's (sender, pulse)
// map, entry i at map[i]); j0 holds the first round's map entries (loaded by
// the caller, possibly before a wait). An empty range touches nothing (its
// sender may hold no slot for the unconditional reads of a round).
// With a staging buffer (the host-orchestrated baseline), entry i of a map
// goes to / comes from stage[map_off + i] instead of the receiver's region.
// With load_first, the first round's entries are loaded here too (j0 unused).
template <int E, int B, typename I, int STG = 0>
__device__ void coords_range(float* x, const I* map, const DChunk& c, int begin, int end,
                             const int (&j0)[E], float* stage = nullptr, bool load_first = false,
                             float* tile = nullptr)
{
    if (begin >= end)
        return;
    const float* src = x + 3ll * c.src_base;
    float* dst = stage ? stage + 3ll * c.map_off : x + 3ll * c.dst_base;
    if (load_first) {
        int j[E];
        load_map<E, B, I>(map, begin, end, j);
        coords_round<E, B, STG>(src, dst, c, begin, end, j, tile);
    } else {
        coords_round<E, B, STG>(src, dst, c, begin, end, j0, tile);
    }
    for (int i0 = begin + B * E; i0 < end; i0 += B * E) {
        int j[E];
        load_map<E, B, I>(map, i0, end, j);
        coords_round<E, B, STG>(src, dst, c, i0, end, j, tile);
    }
}

template <int E, int B, typename I>
__device__ void forces_range(float* f, const I* map, const DChunk& c, int begin, int end,
                             const int (&j0)[E], const float* stage = nullptr,
                             bool load_first = false)
{
    if (begin >= end)
        return;
    float* tgt = f + 3ll * c.src_base;
    const float* from = stage ? stage + 3ll * c.map_off : f + 3ll * c.dst_base;
    if (load_first) {
        int j[E];
        load_map<E, B, I>(map, begin, end, j);
        forces_round<E, B>(from, tgt, begin, end, j);
    } else {
        forces_round<E, B>(from, tgt, begin, end, j0);
    }
    for (int i0 = begin + B * E; i0 < end; i0 += B * E) {
        int j[E];
        load_map<E, B, I>(map, i0, end, j);
        forces_round<E, B>(from, tgt, i0, end, j);
    }
}

// One worker of a fused launch leaves (called by one lane, after the
// worker's records are released when completion flags are on). The last of
// the launch's `workers` to leave sees every worker's records, re-arms the
// ticket and exit counters for the next launch, and publishes the passes the
// launch completed: the fused pass counters and, with completion flags on,
// every pulse's flag ("Dependency-aware packing": the last arrival stores the
// flag).
__device__ void leave_launch(const XArgs& a, uint32_t workers, uint32_t px, uint32_t pf)
{
    const bool publish = a.flags != nullptr;
    const uint32_t old = __hip_atomic_fetch_add(a.ctrl + kCtrlDone, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old != workers - 1u)
        return;
    if (publish)
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
    st_relaxed(a.ctrl + kCtrlTicket, 0u);
    st_relaxed(a.ctrl + kCtrlDone, 0u);
    if (a.nx > 0) {
        st_relaxed(a.ctrl + kCtrlPassX, px);
        if (publish) {
            const uint32_t e = ld_relaxed(a.ctrl + kCtrlEpochX) + 1u;
            for (int q = 0; q < a.P; q++)
                st_relaxed(a.flags + q, e);
            st_relaxed(a.ctrl + kCtrlEpochX, e);
        }
    }
    if (a.nf > 0) {
        st_relaxed(a.ctrl + kCtrlPassF, pf);
        if (publish) {
            const uint32_t e = ld_relaxed(a.ctrl + kCtrlEpochF) + 1u;
            for (int q = 0; q < a.P; q++)
                st_relaxed(a.flags + DDH_MAX_PULSES + q, e);
            st_relaxed(a.ctrl + kCtrlEpochF, e);
        }
    }
}

__device__ __forceinline__ int claim_ticket(const XArgs& a)
{
    const int t = (int)__hip_atomic_fetch_add(a.ctrl + kCtrlTicket, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    return a.static_first ? t + (int)gridDim.x : t;
}

// Thread 0 does every cross-work-group step (ticket claims, waits, chunk
// completion); each of those thread-0 regions is closed by a work-group
// barrier inside the same loop iteration. The region that finishes a chunk
// also claims the next ticket, so no divergent region ever spans the loop's
// back edge: a region that did (finish at the end of one iteration, claim at
// the start of the next) lets the compiler park lane 0 outside the loop while
// the other lanes pass the barrier and re-read a stale ticket forever.
template <int E, int B, typename I, int STG = 0>
__global__ __launch_bounds__(B) void exchange_kernel(XArgs a)
{
    __shared__ int s_ticket;
    // STG: coordinate stores staged through each wavefront's LDS tile, as
    // in the per-pulse kernel (1: register gathers, 2: LDS loads)
    constexpr int kTile = STG == 2 ? E * kDmaTile : STG == 1 ? E * kStageTile : 0;
    __shared__ __align__(16) float stile[STG ? B / 64 * kTile : 1];
    float* tile = STG ? stile + (((int)threadIdx.x >> 6) * kTile) : nullptr;
    const I* maps = static_cast<const I*>(a.maps);
    const int P = a.P;
    const int nt = a.nx + a.nf;
    const uint32_t bump = a.force_timeout ? 0x40000000u : 0u;  // a value nobody reaches
    const uint32_t px = ld_relaxed(a.ctrl + kCtrlPassX) + (a.nx > 0 ? 1u : 0u);
    const uint32_t pf = ld_relaxed(a.ctrl + kCtrlPassF) + 1u;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x) >> 6;  // uniform: 0 in wave 0

    int ntr = 0;         // trace records written by thread 0
    bool held = false;   // this work-group wrote records it has not released
                         // (uniform: every thread tracks the same chunks)
    if (threadIdx.x == 0) {
        trace_rec(a, ntr, kTrStart, gridDim.x);
        s_ticket = a.static_first ? (int)blockIdx.x : claim_ticket(a);
    }
    __syncthreads();
    for (;;) {
        const int t = __builtin_amdgcn_readfirstlane(s_ticket);
        if (t >= nt)
            break;
        if (threadIdx.x == 0)
            trace_rec(a, ntr, kTrClaim, (uint32_t)t);
        if (t < a.nx) {
            const DChunk c = load_chunk(a.xchunks, t);
            // the guide's two-pass pack at work-group level: the independent
            // slice goes out first; the map entries of the dependent slice
            // are loaded before the wait, its records packed after it
            int jh[E], jt[E];
            load_map<E, B, I>(maps + c.map_off, c.hb, c.he, jh);
            load_map<E, B, I>(maps + c.map_off, c.tb, c.te, jt);
            coords_range<E, B, I, STG>(a.x, maps + c.map_off, c, c.hb, c.he, jh, nullptr, false,
                                       tile);
            if (c.wait_a) {
                if (wave == 0) {
                    if (threadIdx.x == 0)
                        trace_rec(a, ntr, kTrHead, (uint32_t)(c.he - c.hb));
                    wave_wait(a, a.xcnt, a.xneed, px, c.wait_a, c.S * P, 0u, 0, bump);
                    if (threadIdx.x == 0)
                        trace_rec(a, ntr, kTrWaited, c.wait_a);
                }
                __syncthreads();
            }
            coords_range<E, B, I, STG>(a.x, maps + c.map_off, c, c.tb, c.te, jt, nullptr, false,
                                       tile);
            // every wave's records are in L2 before thread 0 releases them
            if (c.flags & kChunkRelease)
                wait_vm_idle();
            held = !(c.flags & kChunkRelease);
            __syncthreads();
            if (threadIdx.x == 0) {
                trace_rec(a, ntr, kTrChunk, (uint32_t)(c.he - c.hb + c.te - c.tb));
                if (c.flags & kChunkRelease)
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                add_relaxed(a.xcnt + c.ctr, 1u);
                trace_rec(a, ntr, kTrPublish, (uint32_t)c.ctr);
                s_ticket = claim_ticket(a);
            }
            __syncthreads();
        } else {
            const DChunk c = load_chunk(a.fchunks, t - a.nx);
            int j0[E];
            load_map<E, B, I>(maps + c.map_off, c.hb, c.he, j0);  // static: before any wait
            // a step's force chunks do not wait for its coordinate chunks:
            // the passes touch different arrays
            if (c.wait_a || c.wait_b) {
                if (wave == 0) {
                    wave_wait(a, a.fcnt, a.fneed, pf, c.wait_a, c.S * P, c.wait_b, c.R * P, bump);
                    if (threadIdx.x == 0)
                        trace_rec(a, ntr, kTrWaited, c.wait_a | (c.wait_b << 16));
                }
                __syncthreads();
            }
            forces_range<E, B, I>(a.f, maps + c.map_off, c, c.hb, c.he, j0);
            // every wave's sums are in L2 before thread 0 releases them
            if (c.flags & kChunkRelease)
                wait_vm_idle();
            held = !(c.flags & kChunkRelease);
            __syncthreads();
            if (threadIdx.x == 0) {
                trace_rec(a, ntr, kTrChunk, (uint32_t)(c.he - c.hb));
                if (c.flags & kChunkRelease)
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                add_relaxed(a.fcnt + c.ctr, 1u);
                trace_rec(a, ntr, kTrPublish, (uint32_t)(0x10000 | c.ctr));
                s_ticket = claim_ticket(a);
            }
            __syncthreads();
        }
    }

    // Leave: a work-group that still holds unreleased records (chunks no
    // later chunk of the launch reads) releases them, then leave_launch.
    // (Without completion flags, a.flags is null: nothing to release here.)
    const bool publish = a.flags != nullptr;
    if (held && publish) {
        wait_vm_idle();
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        trace_rec(a, ntr, kTrExit, 0);
        if (held && publish)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        leave_launch(a, gridDim.x, px, pf);
    }
}

// Fused mode at wavefront granularity (DDH_TUNE_WAVE_CHUNKS; the per-warp
// pipelining of the guide's "NVLink path: TMA-based direct stores"): every
// wavefront of the launch is an independent worker and no work-group barrier
// is ever taken. A chunk is one contiguous slice of one map. The wavefront
// claims it, packs the slice's independent entries, waits only if the slice
// also holds dependent entries (the map's tail), packs those, and publishes
// by itself: when a later chunk reads its records, a release fence (which
// waits for the wavefront's own stores and writes them back), then one
// relaxed add to the map's counter. Same ticket order, counters and targets
// as exchange_kernel, hence the same freedom from deadlock; in the exit
// protocol every wavefront counts as one worker.
template <int E, typename I, int STG = 0>
__global__ __launch_bounds__(256) void wave_kernel(XArgs a)
{
    constexpr int W = 64;  // lanes that share a round: one wavefront
    // STG: coordinate stores staged through the wavefront's LDS tile, as in
    // the per-pulse kernel (1: register gathers, 2: LDS loads)
    constexpr int kTile = STG == 2 ? E * kDmaTile : STG == 1 ? E * kStageTile : 0;
    __shared__ __align__(16) float stile[STG ? 4 * kTile : 1];
    float* tile = STG ? stile + (((int)threadIdx.x >> 6) * kTile) : nullptr;
    const I* maps = static_cast<const I*>(a.maps);
    const int P = a.P;
    const int nt = a.nx + a.nf;
    const uint32_t bump = a.force_timeout ? 0x40000000u : 0u;
    const uint32_t px = ld_relaxed(a.ctrl + kCtrlPassX) + (a.nx > 0 ? 1u : 0u);
    const uint32_t pf = ld_relaxed(a.ctrl + kCtrlPassF) + 1u;
    const bool lead = (threadIdx.x & 63) == 0;
    bool held = false;   // this wavefront wrote records it has not released
    for (;;) {
        int t = 0;
        if (lead)
            t = (int)__hip_atomic_fetch_add(a.ctrl + kCtrlTicket, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        t = __builtin_amdgcn_readfirstlane(t);  // lane 0's (every lane is active)
        if (t >= nt)
            break;
        if (t < a.nx) {
            const DChunk c = load_chunk(a.xchunks, t);
            int jh[E], jt[E];
            load_map<E, W, I>(maps + c.map_off, c.hb, c.he, jh);
            load_map<E, W, I>(maps + c.map_off, c.tb, c.te, jt);
            coords_range<E, W, I, STG>(a.x, maps + c.map_off, c, c.hb, c.he, jh, nullptr, false,
                                       tile);
            if (c.wait_a)
                wave_wait(a, a.xcnt, a.xneed, px, c.wait_a, c.S * P, 0u, 0, bump);
            coords_range<E, W, I, STG>(a.x, maps + c.map_off, c, c.tb, c.te, jt, nullptr, false,
                                       tile);
            if (c.flags & kChunkRelease)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            held = !(c.flags & kChunkRelease);
            // the lanes of a wavefront run in lockstep, so every lane's
            // stores and fence precede lane 0's add; the wave barrier keeps
            // the compiler from moving anything across it
            __builtin_amdgcn_wave_barrier();
            if (lead)
                add_relaxed(a.xcnt + c.ctr, 1u);
        } else {
            const DChunk c = load_chunk(a.fchunks, t - a.nx);
            int j0[E];
            load_map<E, W, I>(maps + c.map_off, c.hb, c.he, j0);
            if (c.wait_a || c.wait_b)
                wave_wait(a, a.fcnt, a.fneed, pf, c.wait_a, c.S * P, c.wait_b, c.R * P, bump);
            forces_range<E, W, I>(a.f, maps + c.map_off, c, c.hb, c.he, j0);
            if (c.flags & kChunkRelease)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            held = !(c.flags & kChunkRelease);
            __builtin_amdgcn_wave_barrier();
            if (lead)
                add_relaxed(a.fcnt + c.ctr, 1u);
        }
    }
    const bool publish = a.flags != nullptr;
    if (held && publish)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_wave_barrier();
    if (lead)
        leave_launch(a, gridDim.x * (blockDim.x / 64), px, pf);
}

// One pulse of one pass, ordered against the other pulses by the stream
// alone: chunk b of the launch (blocks take b, b + grid, ...) is coordinate
// chunk xbegin + b for b < nxb, else force chunk fbegin + b - nxb. A step call pairs coordinate pulse q with force
// pulse P-1-q in one launch (the two passes touch different arrays, and each
// pair's predecessors are complete at the launch boundary). No tickets,
// counters, waits or fences: the kernel boundary publishes the writes.
struct PArgs {
    float* x;
    float* f;
    const void* pad;   // chunk-aligned map entries in the kernel's index type,
                       // or null: entries come from maps after the descriptor
    const void* maps;  // the maps in the kernel's index type
    int32_t chunk;     // entries per chunk slot of pad
    int32_t xpad;      // pad slot of the launch's first coordinate chunk
    int32_t fpad;      // pad slot of the launch's first force chunk
    const DChunk* xchunks;
    const DChunk* fchunks;
    int32_t xbegin, nxb, fbegin;
    int32_t nb;       // chunks of the launch (blocks loop over them)
    int32_t xgroup;   // neighbouring chunks per XCD turn (0: a contiguous
                      // eighth of the chunks per XCD)
    float* stage;     // null, or the staging buffer of the host-orchestrated mode
    uint32_t* ctrl;
    uint32_t* flags;
    uint32_t xdone;   // coordinate / force pulses that earlier launches of the
    uint32_t fdone;   // call completed, whose flags this launch publishes
    uint32_t xexit;   // coordinate / force pulses whose flags this launch
    uint32_t fexit;   // publishes when its last block leaves (0: none)
    int32_t op;       // with xexit / fexit: the passes the call completes
};

// Completion flags of pulses that earlier launches of the same call finished:
// the launch boundary has made their records visible, so relaxed stores of
// the epoch the call is completing suffice.
__device__ __forceinline__ void publish_done(const PArgs& a)
{
    const int q = (int)threadIdx.x;
    if (blockIdx.x == 0 && q < DDH_MAX_PULSES && ((a.xdone | a.fdone) >> q & 1u)) {
        if (a.xdone >> q & 1u)
            st_relaxed(a.flags + q, ld_relaxed(a.ctrl + kCtrlEpochX) + 1u);
        if (a.fdone >> q & 1u)
            st_relaxed(a.flags + DDH_MAX_PULSES + q, ld_relaxed(a.ctrl + kCtrlEpochF) + 1u);
    }
}

// The last block of a launch that publishes its own pulses' flags: every
// block waits for its waves' stores, releases them (agent scope) and counts
// itself out; the block that counts last acquires every other block's
// records and stores the flags and the epochs of the passes the call
// completes, then re-arms the count for the next such launch.
__device__ void exit_publish(const PArgs& a)
{
    wait_vm_idle();
    __syncthreads();
    if (threadIdx.x != 0)
        return;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = __hip_atomic_fetch_add(a.ctrl + kCtrlPulseDone, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old != gridDim.x - 1u)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
    st_relaxed(a.ctrl + kCtrlPulseDone, 0u);
    const uint32_t ex = ld_relaxed(a.ctrl + kCtrlEpochX) + 1u;
    const uint32_t ef = ld_relaxed(a.ctrl + kCtrlEpochF) + 1u;
    for (int q = 0; q < DDH_MAX_PULSES; q++) {
        if (a.xexit >> q & 1u)
            st_relaxed(a.flags + q, ex);
        if (a.fexit >> q & 1u)
            st_relaxed(a.flags + DDH_MAX_PULSES + q, ef);
    }
    if (a.op & kOpCoords)
        st_relaxed(a.ctrl + kCtrlEpochX, ex);
    if (a.op & kOpForces)
        st_relaxed(a.ctrl + kCtrlEpochF, ef);
}

// The loads that start chunk b of a per-pulse launch: its descriptor and
// its first round's map entries (raw: entries past the chunk's end are
// masked once the descriptor is in). With the pad, the entries come from the
// chunk's pad slot, located by the chunk index alone, so their loads issue
// before the descriptor arrives (the pad holds zeros past every chunk and
// after the last one, so the loads stay in bounds); without it, from the
// maps, after the descriptor. m receives the chunk's map base (entry i at
// m[i]).
template <int E, int B, typename I>
__device__ __forceinline__ void pulse_fetch(const PArgs& a, int b, DChunk& c, int (&j)[E],
                                            const I*& m)
{
    const bool xs = b < a.nxb;
    const I* pad = static_cast<const I*>(a.pad);
    if (pad) {
        const I* slot = pad + (int64_t)(xs ? a.xpad + b : a.fpad + (b - a.nxb)) * a.chunk;
#pragma unroll
        for (int e = 0; e < E; e++)
            j[e] = (int)slot[e * B + (int)threadIdx.x];
        c = xs ? load_chunk(a.xchunks, a.xbegin + b) : load_chunk(a.fchunks, a.fbegin + (b - a.nxb));
        m = slot - c.hb;
    } else {
        c = xs ? load_chunk(a.xchunks, a.xbegin + b) : load_chunk(a.fchunks, a.fbegin + (b - a.nxb));
        m = static_cast<const I*>(a.maps) + c.map_off;
        load_map<E, B, I>(m, c.hb, c.he, j);
    }
}

// STG: the coordinate chunks stage their stores through LDS, gathered
// into registers (1, coords_put_lds) or by LDS loads (2, coords_dma_put);
// the force chunks are the same in every form.
template <int E, int B, typename I, int STG = 0>
__global__ __launch_bounds__(B) void pulse_kernel(PArgs a)
{
    constexpr int kTile = STG == 2 ? E * kDmaTile : STG == 1 ? E * kStageTile : 0;
    __shared__ __align__(16) float stile[STG ? B / 64 * kTile : 1];
    float* tile = STG ? stile + (((int)threadIdx.x >> 6) * kTile) : nullptr;
    publish_done(a);
    // Software pipeline over the block's chunks b, b + grid, ...: chunk b's
    // gathers are issued first, then the descriptor and map entries of the
    // block's next chunk, then chunk b's stores, so the next chunk's first
    // loads are in flight while this one's records arrive.
    const int grid = (int)gridDim.x;
    // neighbouring chunks share an XCD: a contiguous eighth of them per XCD
    // where launches are latency-bound (small chunks), else groups of four
    // dealt in turn, so every XCD takes coordinate and force chunks alike
    int b = a.xgroup ? xcd_group<4>((int)blockIdx.x, grid) : xcd_tile((int)blockIdx.x, grid);
    DChunk c;
    int jr[E];
    const I* m = nullptr;
    if (b < a.nb)
        pulse_fetch<E, B, I>(a, b, c, jr, m);
    for (; b < a.nb; b += grid) {
        const DChunk cc = c;
        const I* mc = m;
        int j0[E];
        const int n = cc.he - cc.hb;
#pragma unroll
        for (int e = 0; e < E; e++)
            j0[e] = e * B + (int)threadIdx.x < n ? jr[e] : -1;
        const int bn = b + grid;
        if (n <= 0) {
            // an empty map's chunk: nothing to move (its sender or region
            // may hold no slot to read)
            if (bn < a.nb)
                pulse_fetch<E, B, I>(a, bn, c, jr, m);
        } else if (b < a.nxb) {
            const float* src = a.x + 3ll * cc.src_base;
            float* dst = a.stage ? a.stage + 3ll * cc.map_off : a.x + 3ll * cc.dst_base;
            if constexpr (STG == 2) {
                coords_dma_issue<E>(src, j0, tile);
                if (bn < a.nb)
                    pulse_fetch<E, B, I>(a, bn, c, jr, m);
                coords_dma_put<E, B>(dst, cc, cc.hb, cc.he, tile);
            } else {
                float v[E][3];
                coords_gather<E, B>(src, j0, v);
                if (bn < a.nb)
                    pulse_fetch<E, B, I>(a, bn, c, jr, m);
                if constexpr (STG == 1)
                    coords_put_lds<E, B>(dst, cc, cc.hb, cc.he, v, tile);
                else
                    coords_put<E, B>(dst, cc, cc.hb, cc.he, v);
            }
            if (n > E * B)
                coords_range<E, B, I, STG>(a.x, mc, cc, cc.hb + E * B, cc.he, j0, a.stage, true,
                                           tile);
        } else {
            float* tgt = a.f + 3ll * cc.src_base;
            const float* from = a.stage ? a.stage + 3ll * cc.map_off : a.f + 3ll * cc.dst_base;
            float sv[E][3], tv[E][3];
            forces_gather<E, B>(from, tgt, cc.hb, j0, sv, tv);
            if (bn < a.nb)
                pulse_fetch<E, B, I>(a, bn, c, jr, m);
            forces_put<E, B>(tgt, j0, sv, tv);
            if (n > E * B)
                forces_range<E, B, I>(a.f, mc, cc, cc.hb + E * B, cc.he, j0, a.stage, true);
        }
    }
    if (a.xexit | a.fexit)
        exit_publish(a);
}

// After the launches of a call (stream-ordered, so complete): the completion
// flags of the pulses in xmask / fmask not published yet, then the epochs of
// the passes the call completed (op: kOpCoords / kOpForces bits).
__global__ void signal_kernel(uint32_t* ctrl, uint32_t* flags, uint32_t xmask, uint32_t fmask,
                              int op)
{
    const int q = threadIdx.x;
    const uint32_t ex = ld_relaxed(ctrl + kCtrlEpochX) + 1u;
    const uint32_t ef = ld_relaxed(ctrl + kCtrlEpochF) + 1u;
    if (q < DDH_MAX_PULSES) {
        if (xmask >> q & 1u)
            st_relaxed(flags + q, ex);
        if (fmask >> q & 1u)
            st_relaxed(flags + DDH_MAX_PULSES + q, ef);
    }
    __syncthreads();
    if (q == 0) {
        if (op & kOpCoords)
            st_relaxed(ctrl + kCtrlEpochX, ex);
        if (op & kOpForces)
            st_relaxed(ctrl + kCtrlEpochF, ef);
    }
}

// One wave waits until flags[idx] reaches epoch (modulo 2^32), then
// acquires, so the work enqueued after it on the same stream sees every
// record the flag covers. Bounded by the spin limit (DDH_ETIMEOUT).
__global__ void wait_flag_kernel(const uint32_t* flags, int idx, uint32_t epoch, uint32_t* ctrl,
                                 uint32_t spin_limit)
{
    uint32_t n = 0;
    for (;;) {
        const bool ok = (int32_t)(ld_relaxed(flags + idx) - epoch) >= 0;
        if (__all(ok))
            break;
        if (++n >= spin_limit) {
            if (threadIdx.x == 0) {
                uint32_t zero = 0;
                __hip_atomic_compare_exchange_strong(ctrl + kCtrlError, &zero,
                                                     (uint32_t)DDH_ETIMEOUT, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// x_local[home_slot[r]] = x_global[home_gid[r]] for every home atom r.
__global__ __launch_bounds__(kBlock) void gather_home_kernel(const float* __restrict__ xg,
                                                             float* __restrict__ x,
                                                             const int32_t* __restrict__ gid,
                                                             const int32_t* __restrict__ slot,
                                                             int32_t n)
{
    const int r = blockIdx.x * kBlock + threadIdx.x;
    if (r >= n)
        return;
    const float* s = xg + 3ll * gid[r];
    float* d = x + 3ll * slot[r];
    d[0] = s[0];
    d[1] = s[1];
    d[2] = s[2];
}

bool use_narrow_maps(const Plan* p) { return p->narrow_maps && p->d_maps16; }

// The fused kernel instance for the work-group width and entries per lane.
template <typename I>
void launch_fused_t(const XArgs& a, int grid, bool wide, int per, int stg, hipStream_t s)
{
    if (stg && wide) {  // 1024 lanes; the staged forms are built for the wide block only
        if (per > 2)
            hipLaunchKernelGGL((stg == 1 ? exchange_kernel<4, 1024, I, 1> : exchange_kernel<4, 1024, I, 2>),
                               dim3(grid), dim3(1024), 0, s, a);
        else if (per > 1)
            hipLaunchKernelGGL((stg == 1 ? exchange_kernel<2, 1024, I, 1> : exchange_kernel<2, 1024, I, 2>),
                               dim3(grid), dim3(1024), 0, s, a);
        else
            hipLaunchKernelGGL((stg == 1 ? exchange_kernel<1, 1024, I, 1> : exchange_kernel<1, 1024, I, 2>),
                               dim3(grid), dim3(1024), 0, s, a);
    } else if (wide) {
        if (per > 2)
            hipLaunchKernelGGL((exchange_kernel<4, 1024, I>), dim3(grid), dim3(1024), 0, s, a);
        else if (per > 1)
            hipLaunchKernelGGL((exchange_kernel<2, 1024, I>), dim3(grid), dim3(1024), 0, s, a);
        else
            hipLaunchKernelGGL((exchange_kernel<1, 1024, I>), dim3(grid), dim3(1024), 0, s, a);
    } else {
        if (per > 8)
            hipLaunchKernelGGL((exchange_kernel<16, 256, I>), dim3(grid), dim3(256), 0, s, a);
        else if (per > 4)
            hipLaunchKernelGGL((exchange_kernel<8, 256, I>), dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((exchange_kernel<4, 256, I>), dim3(grid), dim3(256), 0, s, a);
    }
}

// The wavefront-granular fused kernel for the entries per lane.
template <typename I>
void launch_wave_t(const XArgs& a, int grid, int per, int stg, hipStream_t s)
{
    if (per > 4)
        hipLaunchKernelGGL((stg == 2 ? wave_kernel<8, I, 2> : stg == 1 ? wave_kernel<8, I, 1>
                                                                       : wave_kernel<8, I, 0>),
                           dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((stg == 2 ? wave_kernel<4, I, 2> : stg == 1 ? wave_kernel<4, I, 1>
                                                                       : wave_kernel<4, I, 0>),
                           dim3(grid), dim3(256), 0, s, a);
}

// The per-pulse kernel instance for the block width and entries per lane.
template <typename I>
void launch_pulse_t(const PArgs& a, dim3 grid, int lanes, int per, int stg, hipStream_t s)
{
    const dim3 block(lanes);
    if (stg == 1) {  // 256 lanes, at most eight entries per lane and round (sixteen spill)
        if (per > 4)
            hipLaunchKernelGGL((pulse_kernel<8, 256, I, 1>), grid, block, 0, s, a);
        else if (per > 2)
            hipLaunchKernelGGL((pulse_kernel<4, 256, I, 1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((pulse_kernel<2, 256, I, 1>), grid, block, 0, s, a);
    } else if (stg == 2) {
        if (per > 4)
            hipLaunchKernelGGL((pulse_kernel<8, 256, I, 2>), grid, block, 0, s, a);
        else if (per > 2)
            hipLaunchKernelGGL((pulse_kernel<4, 256, I, 2>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((pulse_kernel<2, 256, I, 2>), grid, block, 0, s, a);
    } else if (lanes == 512) {
        if (per > 4)
            hipLaunchKernelGGL((pulse_kernel<8, 512, I>), grid, block, 0, s, a);
        else if (per > 2)
            hipLaunchKernelGGL((pulse_kernel<4, 512, I>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((pulse_kernel<2, 512, I>), grid, block, 0, s, a);
    } else if (lanes == 1024) {
        if (per > 2)
            hipLaunchKernelGGL((pulse_kernel<4, 1024, I>), grid, block, 0, s, a);
        else if (per > 1)
            hipLaunchKernelGGL((pulse_kernel<2, 1024, I>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((pulse_kernel<1, 1024, I>), grid, block, 0, s, a);
    } else {
        if (per > 8)
            hipLaunchKernelGGL((pulse_kernel<16, 256, I>), grid, block, 0, s, a);
        else if (per > 4)
            hipLaunchKernelGGL((pulse_kernel<8, 256, I>), grid, block, 0, s, a);
        else if (per > 2)
            hipLaunchKernelGGL((pulse_kernel<4, 256, I>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((pulse_kernel<2, 256, I>), grid, block, 0, s, a);
    }
}

int launch_fused(const Plan* p, XArgs a, hipStream_t s)
{
    const int nt = a.nx + a.nf;
    if (nt <= 0)
        return DDH_OK;
    if (p->fused.wave) {
        // work-groups of four independent wavefronts, at most eight per
        // compute unit and one wavefront per ticket
        int grid = p->grid_req > 0 ? p->grid_req : p->n_cu * 8;
        grid = std::min(grid, (nt + 3) / 4);
        a.static_first = 0;
        const int per = (p->fused.chunk + 63) / 64;
        if (use_narrow_maps(p)) {
            a.maps = p->d_maps16;
            launch_wave_t<uint16_t>(a, grid, per, p->lds_stage, s);
        } else {
            a.maps = p->d_maps;
            launch_wave_t<int32_t>(a, grid, per, p->lds_stage, s);
        }
        DDH_HIP(hipGetLastError());
        return DDH_OK;
    }
    // one 1024-wide work-group per compute unit: fewer work-groups mean fewer
    // serialized ticket claims and exit releases (1M atoms: 54.8 -> 42.1 us
    // per fused step against four 256-wide work-groups per compute unit;
    // 384k: 98.8 -> 78.2; 12M: 343 -> 316)
    int grid = p->grid_req > 0 ? p->grid_req : p->n_cu;
    if (grid > nt)
        grid = nt;
    // Tickets are claimed in the order work-groups start, so a chunk only
    // waits on chunks whose work-groups are already running, whatever else
    // shares the GPU. On request (the caller guarantees the launch has the
    // GPU to itself) a grid of at most one work-group per compute unit lets
    // work-group b start with ticket b unclaimed; a concurrent kernel that
    // holds compute units could then leave a producer undispatched behind
    // its consumers.
    a.static_first = (p->static_first && grid <= p->n_cu) ? 1 : 0;
    // work-group width 1024 unless requested otherwise; entries per lane and
    // round from the chunk size
    const bool wide = p->block_req ? p->block_req == 1024 : true;
    const int per = (p->fused.chunk + (wide ? 1023 : 255)) / (wide ? 1024 : 256);
    if (use_narrow_maps(p)) {
        a.maps = p->d_maps16;
        launch_fused_t<uint16_t>(a, grid, wide, per, p->lds_stage, s);
    } else {
        a.maps = p->d_maps;
        launch_fused_t<int32_t>(a, grid, wide, per, p->lds_stage, s);
    }
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

// Coordinate chunks [xb, xe) and force chunks [fb, fe) of table t in one
// launch; entries per lane and round from the table's chunk size (larger
// chunks take several rounds).
// xdone / fdone: pulses completed by earlier launches of the call whose flags
// this launch publishes; cleared when the launch takes them over.
// Whether blocks read the chunk-aligned map copy (their first map loads
// issue before the descriptor arrives) or the maps themselves after it (no
// reads of the copy's padding).
bool use_pad_maps(const Plan* p)
{
    if (p->pad_maps)
        return p->pad_maps == 1;
    return true;
}

// Whether the call's last per-pulse launch publishes its own flags at exit
// (every block releases, the last one stores the flags) rather than a
// one-wave launch after it.
bool use_exit_publish(const Plan* p)
{
    if (p->exit_publish)
        return p->exit_publish == 1;
    return false;
}

// xexit / fexit / op: pulses whose flags the launch publishes when its last
// block leaves, and the passes the call completes (0: none). *launched tells
// whether the launch had any chunk (an empty launch is not enqueued).
int launch_pulse(const Plan* p, float* x, float* f, const WorkTable& t, int xb, int xe, int fb,
                 int fe, hipStream_t s, uint32_t& xdone, uint32_t& fdone, float* stage = nullptr,
                 uint32_t xexit = 0u, uint32_t fexit = 0u, int op = 0, bool* launched = nullptr)
{
    const int nb = (xe - xb) + (fe - fb);
    if (launched)
        *launched = nb > 0;
    if (nb <= 0)
        return DDH_OK;
    PArgs a{};
    a.x = x;
    a.f = f;
    const bool narrow = use_narrow_maps(p);
    a.pad = !use_pad_maps(p) ? nullptr : narrow ? (const void*)t.d_pad16 : (const void*)t.d_pad;
    a.maps = narrow ? (const void*)p->d_maps16 : (const void*)p->d_maps;
    a.chunk = t.chunk;
    a.xgroup = t.chunk > kSmallChunk ? 4 : 0;
    // pad slots: coordinate chunk k owns slot k; a force chunk uses the slot
    // of the coordinate chunk of the same map slice (the tables slice every
    // map alike, and list a pulse's chunks in the same order in both passes)
    a.xpad = xb;
    a.fpad = 0;
    if (fe > fb) {
        const int P = p->g.P;
        int r = 0;
        while (r + 1 < P && t.fpulse_begin[r + 1] <= fb)
            r++;
        a.fpad = t.xpulse_begin[P - 1 - r] + (fb - t.fpulse_begin[r]);
    }
    a.xchunks = t.d_xch;
    a.fchunks = t.d_fch;
    a.xbegin = xb;
    a.nxb = xe - xb;
    a.fbegin = fb;
    a.stage = stage;
    a.ctrl = p->d_ctrl;
    a.flags = p->d_pflag;
    a.xdone = p->flags ? xdone : 0u;
    a.fdone = p->flags ? fdone : 0u;
    xdone = fdone = 0u;
    a.xexit = p->flags ? xexit : 0u;
    a.fexit = p->flags ? fexit : 0u;
    a.op = op;
    // 256-wide blocks by default, with up to sixteen entries per lane and
    // round: each lane issues its gathers back to back, and the compute units
    // hold eight blocks each (12M atoms: 111.4 us per step against 114.5 with
    // 1024-wide blocks and two entries per lane; 384k: 22.8 against 27.4)
    const int lanes = p->block_req ? p->block_req : 256;
    const int per = (t.chunk + lanes - 1) / lanes;
    // at most the blocks the compute units hold at once; each loops over the
    // launch's chunks (A/B on MI355X: 96k 9.46 -> 9.22 us, 12M 119.5 -> 118.7)
    a.nb = nb;
    const int resident = p->n_cu * (2048 / lanes);
    const dim3 grid(std::min(nb, resident));
    const int stg = lanes == 256 && a.nxb > 0 ? p->lds_stage : 0;
    if (narrow)
        launch_pulse_t<uint16_t>(a, grid, lanes, per, stg, s);
    else
        launch_pulse_t<int32_t>(a, grid, lanes, per, stg, s);
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

// The launches of one call in mode (FUSED or PULSE), enqueued on s.
int enqueue_raw(Plan* p, int op, float* x, float* f, hipStream_t s, int mode)
{
    const int P = p->g.P;
    if (!(mode & DDH_MODE_PULSE)) {
        // made at the build, or by ddh_set_mode, whenever the mode may
        // resolve to the fused launch
        if (!p->fused_ready)
            return fail(DDH_ESTATE, "the fused launch's table was not made for this build");
        XArgs a{};
        a.x = x;
        a.f = f;
        const WorkTable& t = p->fused;
        a.xchunks = t.d_xch;
        a.fchunks = t.d_fch;
        a.nx = (op & kOpCoords) ? (int)t.xch.size() : 0;
        a.nf = (op & kOpForces) ? (int)t.fch.size() : 0;
        a.ctrl = p->d_ctrl;
        a.xcnt = p->d_xcnt;
        a.fcnt = p->d_fcnt;
        a.xneed = p->d_xneed;
        a.fneed = p->d_fneed;
        a.P = P;
        a.force_timeout = p->force_timeout;
        a.spin_limit = p->spin_limit;
        a.trace = p->trace;
        a.flags = p->flags ? p->d_pflag : nullptr;
        return launch_fused(p, a, s);
    }
    // one launch per pulse: coordinates in increasing, forces in decreasing
    // pulse order (fpulse_begin is already in that order); a step pairs the
    // q-th launch of each pass. Launch q publishes the flags of launch q-1's
    // pulses; a last one-wave launch those of the final launch.
    const WorkTable& t = p->pulse_table(op);
    const auto& xb = t.xpulse_begin;
    const auto& fb = t.fpulse_begin;
    const bool xs = op & kOpCoords, fs = op & kOpForces;
    const bool exit_pub = p->flags && use_exit_publish(p);
    int rc = DDH_OK;
    uint32_t xdone = 0u, fdone = 0u;  // completed pulses whose flags are pending
    for (int q = 0; q < P && !rc; q++) {
        const uint32_t xq = xs ? 1u << q : 0u, fq = fs ? 1u << (P - 1 - q) : 0u;
        if (exit_pub && q == P - 1) {
            // the last launch publishes its own pulses when its last block
            // leaves (those still pending from earlier launches at its start)
            bool launched = false;
            rc = launch_pulse(p, x, f, t, xs ? xb[q] : 0, xs ? xb[q + 1] : 0, fs ? fb[q] : 0,
                              fs ? fb[q + 1] : 0, s, xdone, fdone, nullptr, xq, fq, op,
                              &launched);
            if (!rc && launched)
                return DDH_OK;
            // an empty last launch: the one-wave launch below publishes
            xdone |= xq;
            fdone |= fq;
            break;
        }
        rc = launch_pulse(p, x, f, t, xs ? xb[q] : 0, xs ? xb[q + 1] : 0, fs ? fb[q] : 0,
                          fs ? fb[q + 1] : 0, s, xdone, fdone);
        xdone |= xq;
        fdone |= fq;
    }
    if (rc || !p->flags)
        return rc;
    hipLaunchKernelGGL(signal_kernel, dim3(1), dim3(64), 0, s, p->d_ctrl, p->d_pflag, xdone, fdone,
                       op);
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

// The host-orchestrated baseline ("From MPI baseline to optimized GPU-native
// halo exchange": pack, hand the buffer to the host, send and receive, then
// unpack; two blocking waits per pulse). Per coordinate pulse: one pack
// launch into the staging buffer, a host wait, one device-to-device copy per
// sender into the receiver's region, a host wait. Per force pulse (reverse
// order): one copy per sender of the receiver's region into the staging
// buffer, a host wait, one unpack launch that adds, a host wait. The staging
// buffer holds every map entry once (entry i of map (S, p) at map_off + i).
// stage: a device buffer of at least 3 * n_halo floats.
int enqueue_staged(Plan* p, int op, float* x, float* f, hipStream_t s, float* stage)
{
    const int P = p->g.P, D = p->g.ndom;
    const WorkTable& t = p->pulse;
    const auto& xb = t.xpulse_begin;
    const auto& fb = t.fpulse_begin;
    uint32_t none = 0u;  // the flags are published once, at the end of the call
    auto copies = [&](int q, float* arr, bool to_region) -> int {
        for (int S = 0; S < D; S++) {
            const int it = S * P + q;
            const size_t n = (size_t)p->send[it];
            if (n == 0)
                continue;
            float* region = arr + 3 * (p->base[p->recv[it]] + p->roff[it]);
            float* staged = stage + 3 * p->map_off[it];
            DDH_HIP(hipMemcpyAsync(to_region ? region : staged, to_region ? staged : region,
                                   sizeof(float) * 3 * n, hipMemcpyDeviceToDevice, s));
        }
        return DDH_OK;
    };
    int rc = DDH_OK;
    if (op & kOpCoords)
        for (int q = 0; q < P; q++) {
            if ((rc = launch_pulse(p, x, f, t, xb[q], xb[q + 1], 0, 0, s, none, none, stage)))
                return rc;
            DDH_HIP(hipStreamSynchronize(s));
            if ((rc = copies(q, x, true)))
                return rc;
            DDH_HIP(hipStreamSynchronize(s));
        }
    if (op & kOpForces)
        for (int r = 0; r < P; r++) {
            if ((rc = copies(P - 1 - r, f, false)))
                return rc;
            DDH_HIP(hipStreamSynchronize(s));
            if ((rc = launch_pulse(p, x, f, t, 0, 0, fb[r], fb[r + 1], s, none, none, stage)))
                return rc;
            DDH_HIP(hipStreamSynchronize(s));
        }
    if (!p->flags)
        return DDH_OK;
    const uint32_t all = (P >= 32 ? 0u : (1u << P)) - 1u;
    hipLaunchKernelGGL(signal_kernel, dim3(1), dim3(64), 0, s, p->d_ctrl, p->d_pflag,
                       (op & kOpCoords) ? all : 0u, (op & kOpForces) ? all : 0u, op);
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

}  // namespace

int enqueue_exchange(Plan* p, int op, float* x, float* f, hipStream_t s)
{
    if (p->g.P == 0 || p->pulse.nchunks.empty())
        return DDH_OK;
    if (!(p->mode & DDH_MODE_GRAPH)) {
        // a capturing stream means the launches will be replayed from the
        // caller's graph (the legacy null stream is never captured)
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (s && hipStreamIsCapturing(s, &cs) != hipSuccess) {
            (void)hipGetLastError();
            cs = hipStreamCaptureStatusNone;
        }
        const bool captured = cs == hipStreamCaptureStatusActive;
        if (p->mode == DDH_MODE_STAGED) {
            if (captured)
                return fail(DDH_EINVAL, "DDH_MODE_STAGED waits on the host: it cannot be captured");
            // the staging buffer is allocated at the first staged call
            if (!p->d_stage && p->n_halo > 0) {
                DDH_HIP(hipMalloc((void**)&p->d_stage, sizeof(float) * 3 * (size_t)p->n_halo));
                p->owned.push_back(p->d_stage);
            }
            return enqueue_staged(p, op, x, f, s, p->d_stage);
        }
        return enqueue_raw(p, op, x, f, s, p->effective_mode(captured));
    }

    const int mode = p->effective_mode(true);
    const auto key = std::make_tuple(op, (void*)x, (void*)f, mode);
    auto found = p->graphs.find(key);
    if (found == p->graphs.end()) {
        if (!p->capture_stream)
            DDH_HIP(hipStreamCreateWithFlags(&p->capture_stream, hipStreamNonBlocking));
        DDH_HIP(hipStreamBeginCapture(p->capture_stream, hipStreamCaptureModeThreadLocal));
        int rc = enqueue_raw(p, op, x, f, p->capture_stream, mode);
        hipGraph_t graph = nullptr;
        hipError_t e = hipStreamEndCapture(p->capture_stream, &graph);
        if (rc)
            return rc;
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamEndCapture");
        hipGraphExec_t exec = nullptr;
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (e != hipSuccess)
            return hip_fail(e, "hipGraphInstantiate");
        if (p->graphs.size() >= 16) {
            for (auto& kv : p->graphs)
                (void)hipGraphExecDestroy(kv.second);
            p->graphs.clear();
        }
        found = p->graphs.emplace(key, exec).first;
    }
    DDH_HIP(hipGraphLaunch(found->second, s));
    return DDH_OK;
}

// ---- the host-orchestrated exchange without allocation
//
// Its staging buffer lives in the file-scope device array below instead of
// device memory allocated at the first staged call, for callers that cannot
// allocate. Each device that loads the library holds one copy of the array
// until the process ends. In host code the array's name is only a host-side
// stand-in: kernels and copies get its per-device address, resolved once per
// device with hipGetSymbolAddress while that device is current.
static __device__ __align__(256) unsigned char scratch[kStaticStageBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int enqueue_staged_static(Plan* p, int op, float* x, float* f, hipStream_t s)
{
    const size_t need = sizeof(float) * 3 * (size_t)p->n_halo;
    if (need > kStaticStageBytes)
        return fail(DDH_ECAPACITY, "ddh_exchange_staged_static: the layout's " +
                                       std::to_string(p->n_halo) + " halo entries need " +
                                       std::to_string(need) + " bytes of staging, above the " +
                                       std::to_string(kStaticStageBytes) + "-byte static buffer");
    if (s) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
            (void)hipGetLastError();
            cs = hipStreamCaptureStatusNone;
        }
        if (cs == hipStreamCaptureStatusActive)
            return fail(DDH_EINVAL,
                        "ddh_exchange_staged_static waits on the host: it cannot be captured");
    }
    int dev = -1;
    DDH_HIP(hipGetDevice(&dev));
    if (dev != p->device)
        return fail(DDH_EINVAL, "ddh_exchange_staged_static: the plan's device must be current");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DDH_EINVAL, "ddh_exchange_staged_static: device index out of range");
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            DDH_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
            g_scratch_ptr[dev] = ptr;
        }
        ptr = g_scratch_ptr[dev];
    }
    if (p->g.P == 0 || p->pulse.nchunks.empty())
        return DDH_OK;
    return enqueue_staged(p, op, x, f, s, static_cast<float*>(ptr));
}

int enqueue_wait_flag(Plan* p, int idx, uint32_t epoch, hipStream_t s)
{
    hipLaunchKernelGGL(wait_flag_kernel, dim3(1), dim3(64), 0, s, p->d_pflag, idx, epoch,
                       p->d_ctrl, p->spin_limit);
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

int enqueue_gather_home(Plan* p, const float* xg, float* x, hipStream_t s)
{
    const int n = p->n_atoms;
    if (n == 0)
        return DDH_OK;
    hipLaunchKernelGGL(gather_home_kernel, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, xg,
                       x, p->d_home_gid, p->d_home_slot, n);
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

}  // namespace ddh
