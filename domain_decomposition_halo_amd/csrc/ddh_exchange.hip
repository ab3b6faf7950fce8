// ddh_exchange.hip - coordinate and force passes of the staged halo exchange
// on gfx950, plus the home-slot gather.
//
// Source ("the guide"): NVIDIA technical blog "A Practical Guide to
// GPU-Initiated Communication for Molecular Dynamics at Scale".
//
// Design on one MI355X. Every domain is a slice of one device array, so the
// guide's direct-store path ("Optimizing for efficient transfers across
// NVIDIA NVLink-connected GPUs") is the only path: a sender gathers its map
// entries and stores them straight into the receiver's slots; nothing is
// staged and nothing is "put". The work of a pass is cut into chunks (an
// entry range of one (sender, pulse) map) listed in a ticket table; a launch
// claims tickets in table order with one atomic per chunk, so a chunk only
// ever waits on chunks claimed before it and the launch cannot deadlock,
// whatever the grid size.
//
//  - Coordinates ("Enabling parallelism across pulses through kernel fusion",
//    "Dependency-aware packing"): the ticket table lists the independent
//    heads of every map first (entries below the sender's home count), in
//    pulse order, then the dependent tails in pulse order. A tail chunk waits
//    until the regions its entries read have been delivered.
//  - Forces ("Force halo exchange: Reversing the dependency chain"): chunks
//    in decreasing pulse order. A chunk of (S, p) adds into slots of S and
//    reads region p of R; it waits until the later pulses that add into the
//    same slots of S, and those that add into R's region p, are done, so each
//    slot receives its adds in decreasing pulse order and the result matches
//    the sequential reverse pass bit for bit.
//  - Completion ("Dependency-aware packing", hierarchical release): each
//    work-group ends a chunk with one agent-scope acq_rel increment of the
//    item's counter; the work-group that completes the item resets the
//    counter and release-stores the pass number into the item's flag. All
//    eight XCDs form one agent, so agent scope plays the role the guide gives
//    to system scope.
//  - Pass numbers: flags hold the number of the pass that set them; the
//    number lives in device memory and the launch that ends a pass publishes
//    it, so flags never need clearing and a captured graph replays as is.
//  - Every wait is bounded by a spin limit; on expiry the wait records
//    DDH_ETIMEOUT in the control block and the work-group carries on, so the
//    launch always drains.
#pragma clang fp contract(off)

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

// Spin until *p == v or the spin limit expires (then record the timeout).
__device__ void wait_eq(const uint32_t* p, uint32_t v, const XArgs& a)
{
    uint32_t n = 0;
    while (ld_relaxed(p) != v) {
        if (++n >= a.spin_limit) {
            uint32_t zero = 0;
            __hip_atomic_compare_exchange_strong(a.ctrl + kCtrlError, &zero,
                                                 (uint32_t)DDH_ETIMEOUT, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// One work-group finished a chunk of an item: count it; the work-group that
// completes the item resets the counter and publishes the item's flag.
__device__ void finish_chunk(uint32_t* cnt, uint32_t nchunks, uint32_t* flag, uint32_t pass,
                             uint32_t* xdone)
{
    uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == nchunks - 1u) {
        st_relaxed(cnt, 0u);
        __hip_atomic_store(flag, pass, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (xdone)
            __hip_atomic_fetch_add(xdone, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Coordinates: x[dst + i] = x[src + map[i]] (+ L on the pulse's component).
// Each thread holds E records: all map loads, then all gathers, then all
// stores, so a wavefront keeps 3E independent memory requests in flight.
template <int E>
__device__ void coords_chunk(const XArgs& a, const DItem& it, int begin, int end)
{
    const int32_t* map = a.maps + it.map_off;
    const float* src = a.x + 3ll * it.src_base;
    float* dst = a.x + 3ll * it.dst_base;
    for (int i0 = begin; i0 < end; i0 += kBlock * E) {
        int j[E];
        float v[E][3];
#pragma unroll
        for (int e = 0; e < E; e++) {
            const int i = i0 + e * kBlock + (int)threadIdx.x;
            j[e] = i < end ? map[i] : -1;
        }
#pragma unroll
        for (int e = 0; e < E; e++) {
            if (j[e] >= 0) {
                const float* s = src + 3ll * j[e];
                v[e][0] = s[0];
                v[e][1] = s[1];
                v[e][2] = s[2];
            }
        }
        // uniform per-component branches keep v[][] in registers
        if (it.do_shift) {
#pragma unroll
            for (int c = 0; c < 3; c++)
                if (it.comp == c) {
#pragma unroll
                    for (int e = 0; e < E; e++)
                        v[e][c] = v[e][c] + it.shift;
                }
        }
#pragma unroll
        for (int e = 0; e < E; e++) {
            const int i = i0 + e * kBlock + (int)threadIdx.x;
            if (i < end) {
                float* d = dst + 3ll * i;
                d[0] = v[e][0];
                d[1] = v[e][1];
                d[2] = v[e][2];
            }
        }
    }
}

// Forces: f[src + map[i]] += f[dst + i] (the receiver's region back into the
// sender's slots).
template <int E>
__device__ void forces_chunk(const XArgs& a, const DItem& it, int begin, int end)
{
    const int32_t* map = a.maps + it.map_off;
    float* tgt = a.f + 3ll * it.src_base;
    const float* from = a.f + 3ll * it.dst_base;
    for (int i0 = begin; i0 < end; i0 += kBlock * E) {
        int j[E];
        float s[E][3], t[E][3];
#pragma unroll
        for (int e = 0; e < E; e++) {
            const int i = i0 + e * kBlock + (int)threadIdx.x;
            j[e] = i < end ? map[i] : -1;
            if (j[e] >= 0) {
                const float* r = from + 3ll * i;
                s[e][0] = r[0];
                s[e][1] = r[1];
                s[e][2] = r[2];
            }
        }
#pragma unroll
        for (int e = 0; e < E; e++) {
            if (j[e] >= 0) {
                const float* q = tgt + 3ll * j[e];
                t[e][0] = q[0];
                t[e][1] = q[1];
                t[e][2] = q[2];
            }
        }
#pragma unroll
        for (int e = 0; e < E; e++) {
            if (j[e] >= 0) {
                float* q = tgt + 3ll * j[e];
                q[0] = t[e][0] + s[e][0];
                q[1] = t[e][1] + s[e][1];
                q[2] = t[e][2] + s[e][2];
            }
        }
    }
}

__device__ __forceinline__ int grab_ticket(const XArgs& a)
{
    return (int)__hip_atomic_fetch_add(a.ctrl + kCtrlTicket, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 does every cross-work-group step (ticket claims, waits, chunk
// completion); each of those thread-0 regions is closed by a work-group
// barrier inside the same loop iteration. The region that finishes a chunk
// also claims the next ticket, so no divergent region ever spans the loop's
// back edge: a region that did (finish at the end of one iteration, claim at
// the start of the next) lets the compiler park lane 0 outside the loop while
// the other lanes pass the barrier and re-read a stale ticket forever.
template <int E>
__global__ __launch_bounds__(kBlock) void exchange_kernel(XArgs a)
{
    __shared__ int s_ticket;
    const uint32_t pass = ld_relaxed(a.ctrl + kCtrlEpoch) + 1u;
    const uint32_t want = a.force_timeout ? pass + 0x40000000u : pass;
    const int nx = a.x_end - a.x_begin;
    const int nt = nx + (a.f_end - a.f_begin);
    const int P = a.P;

    if (threadIdx.x == 0)
        s_ticket = grab_ticket(a);
    __syncthreads();
    for (;;) {
        const int t = __builtin_amdgcn_readfirstlane(s_ticket);
        if (t >= nt)
            break;
        if (t < nx) {
            const DChunk c = a.xchunks[a.x_begin + t];
            const DItem it = a.items[c.item];
            if (c.wait_a) {
                if (threadIdx.x == 0) {
                    for (uint32_t m = c.wait_a; m; m &= m - 1)
                        wait_eq(a.xflag + it.S * P + __builtin_ctz(m), want, a);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                }
                __syncthreads();
            }
            coords_chunk<E>(a, it, c.begin, c.end);
            __syncthreads();
            if (threadIdx.x == 0) {
                finish_chunk(a.xcnt + c.item, (uint32_t)it.nchunks, a.xflag + it.R * P + it.p, pass,
                             a.f_end > a.f_begin ? a.ctrl + kCtrlXDone : nullptr);
                s_ticket = grab_ticket(a);
            }
            __syncthreads();
        } else {
            const DChunk c = a.fchunks[a.f_begin + (t - nx)];
            const DItem it = a.items[c.item];
            if (threadIdx.x == 0) {
                if (nx > 0)
                    wait_eq(a.ctrl + kCtrlXDone,
                            a.force_timeout ? (uint32_t)a.n_items + 0x40000000u : (uint32_t)a.n_items,
                            a);
                for (uint32_t m = c.wait_a; m; m &= m - 1)
                    wait_eq(a.fflag + it.S * P + __builtin_ctz(m), want, a);
                for (uint32_t m = c.wait_b; m; m &= m - 1)
                    wait_eq(a.fflag + it.R * P + __builtin_ctz(m), want, a);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();
            forces_chunk<E>(a, it, c.begin, c.end);
            __syncthreads();
            if (threadIdx.x == 0) {
                finish_chunk(a.fcnt + c.item, (uint32_t)it.nchunks, a.fflag + it.S * P + it.p, pass,
                             nullptr);
                s_ticket = grab_ticket(a);
            }
            __syncthreads();
        }
    }

    // Leave: the last work-group re-arms the ticket counters for the next
    // launch and, if this launch ends a pass, publishes the pass number.
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(a.ctrl + kCtrlDone, 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old == gridDim.x - 1u) {
            st_relaxed(a.ctrl + kCtrlTicket, 0u);
            st_relaxed(a.ctrl + kCtrlDone, 0u);
            st_relaxed(a.ctrl + kCtrlXDone, 0u);
            if (a.bump_epoch)
                __hip_atomic_store(a.ctrl + kCtrlEpoch, pass, __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
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

int entries_per_thread(int chunk)
{
    return chunk >= 4 * kBlock ? 4 : (chunk >= 2 * kBlock ? 2 : 1);
}

int launch(const Plan* p, const XArgs& a, int n_tickets, hipStream_t s)
{
    if (n_tickets <= 0)
        return DDH_OK;
    int grid = p->grid_req > 0 ? p->grid_req : p->n_cu * 8;
    if (grid > n_tickets)
        grid = n_tickets;
    const int E = entries_per_thread(p->chunk);
    if (E == 4)
        hipLaunchKernelGGL(exchange_kernel<4>, dim3(grid), dim3(kBlock), 0, s, a);
    else if (E == 2)
        hipLaunchKernelGGL(exchange_kernel<2>, dim3(grid), dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL(exchange_kernel<1>, dim3(grid), dim3(kBlock), 0, s, a);
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

XArgs base_args(const Plan* p, float* x, float* f)
{
    XArgs a{};
    a.x = x;
    a.f = f;
    a.maps = p->d_maps;
    a.items = p->d_items;
    a.xchunks = (p->mode & DDH_MODE_PULSE) ? p->d_xch_pulse : p->d_xch_fused;
    a.fchunks = p->d_fch;
    a.ctrl = p->d_ctrl;
    a.xflag = p->d_xflag;
    a.fflag = p->d_fflag;
    a.xcnt = p->d_xcnt;
    a.fcnt = p->d_fcnt;
    a.P = p->g.P;
    a.n_items = (int32_t)p->items.size();
    a.force_timeout = p->force_timeout;
    a.spin_limit = p->spin_limit;
    return a;
}

// The launches of one call, enqueued on s.
int enqueue_raw(Plan* p, int op, float* x, float* f, hipStream_t s)
{
    const int P = p->g.P;
    const int nx = (int)p->xch_fused.size();
    const int nf = (int)p->fch.size();
    if (!(p->mode & DDH_MODE_PULSE)) {
        XArgs a = base_args(p, x, f);
        a.bump_epoch = 1;
        if (op & kOpCoords) {
            a.x_begin = 0;
            a.x_end = nx;
        }
        if (op & kOpForces) {
            a.f_begin = 0;
            a.f_end = nf;
        }
        return launch(p, a, (a.x_end - a.x_begin) + (a.f_end - a.f_begin), s);
    }
    // one launch per pulse; the stream orders them, the flags are still set
    std::vector<XArgs> seq;
    if (op & kOpCoords)
        for (int q = 0; q < P; q++) {
            XArgs a = base_args(p, x, f);
            a.x_begin = p->xpulse_begin[q];
            a.x_end = p->xpulse_begin[q + 1];
            seq.push_back(a);
        }
    if (op & kOpForces)
        for (int q = P - 1; q >= 0; q--) {
            XArgs a = base_args(p, x, f);
            a.f_begin = p->fpulse_begin[P - 1 - q];
            a.f_end = p->fpulse_begin[P - q];
            seq.push_back(a);
        }
    for (size_t i = 0; i < seq.size(); i++) {
        seq[i].bump_epoch = (i + 1 == seq.size());
        int rc = launch(p, seq[i], (seq[i].x_end - seq[i].x_begin) + (seq[i].f_end - seq[i].f_begin), s);
        if (rc)
            return rc;
    }
    return DDH_OK;
}

}  // namespace

int enqueue_exchange(Plan* p, int op, float* x, float* f, hipStream_t s)
{
    if (p->g.P == 0 || p->items.empty())
        return DDH_OK;
    if (!(p->mode & DDH_MODE_GRAPH))
        return enqueue_raw(p, op, x, f, s);

    const auto key = std::make_tuple(op, (void*)x, (void*)f, p->mode);
    auto found = p->graphs.find(key);
    if (found == p->graphs.end()) {
        if (!p->capture_stream)
            DDH_HIP(hipStreamCreateWithFlags(&p->capture_stream, hipStreamNonBlocking));
        DDH_HIP(hipStreamBeginCapture(p->capture_stream, hipStreamCaptureModeThreadLocal));
        int rc = enqueue_raw(p, op, x, f, p->capture_stream);
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
