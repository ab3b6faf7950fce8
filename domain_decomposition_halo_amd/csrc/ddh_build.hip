// ddh_build.hip - halo-map builder on gfx950.
//
// Source ("the guide"): NVIDIA technical blog "A Practical Guide to
// GPU-Initiated Communication for Molecular Dynamics at Scale"; the guide
// shows the maps only as inputs of its pack kernels ("From MPI baseline to
// optimized GPU-native halo exchange") and states the relay structure
// ("Accelerating GROMACS using Device-initiated Remote Memory Access") and the
// split of every map at the dependency offset ("Enabling parallelism across
// pulses through kernel fusion"). The selection rule implemented here:
//
//   1. every atom goes to the domain whose half-open interval [b_d[i],
//      b_d[i+1]) holds it in each dimension (fp32 compares decide);
//   2. home atoms of a domain are ordered by sort cell (rows cy + ncy * cz in
//      turn, each a serpentine along x: cell_key), then by class (the first
//      pulses' slab tests, see home_class: a cell that a slab cuts keeps the
//      atoms that pulse sends together), then by global id: a partition of
//      the atoms by domain
//      (block histograms in LDS, one scan, a scatter with LDS counters), a
//      counting sort of each domain's atoms by cell in LDS, then each cell
//      sorted by class and id; or, where a domain or a cell table is too
//      large for LDS, a counting sort over all cells of all domains with
//      device atomics, made deterministic the same way;
//   3. pulse p along d, sender S: candidates are S's home slots and every
//      slot it received in earlier pulses (first pulse of d), or the slots it
//      received in the previous pulse of d (later pulses); slot j is selected
//      iff fl(x_j[d] - lo_d(S)) < rc, and selected slots are compacted in
//      increasing order (wavefront ballots + a work-group prefix). Selected
//      records go to the -d neighbour; a slot is held as (global id, mask of
//      dimensions whose + L shift it carries), so its fp32 coordinate is
//      fl(x + L) or x in each component, exactly what the coordinate pass
//      stores.
//
// The builder runs once per neighbour-search step. It learns the sizes from
// the host's read-back of each pulse's counts (waited for on an event, while
// the pulse's write already runs on the device), and waits for the stream
// after the sort and at the end.
#pragma clang fp contract(off)

#include <algorithm>
#include <cmath>
#include <cstring>

#include "ddh_internal.h"

namespace ddh {

namespace {

constexpr int kScanBlock = 1024;  // elements per scan block (4 per thread)
constexpr int kSelTile = 1024;    // candidate slots per block of the slab selection
// the partition sort: its first two passes (256 threads) take the largest
// of 16, 4 and 1 atoms per thread that still gives at least kPartMinBlocks
// blocks; its LDS tables hold up to kPartMaxDomains domains and
// kPartMaxCells sort cells per domain
constexpr int kPartMinBlocks = 512;
constexpr int kPartMaxDomains = 2048;
constexpr int kPartMaxCells = 4096;
constexpr int kDomCap = 32768;           // atoms of a domain sorted in LDS
constexpr int kDomBatch = 8;             // record loads a thread issues together
// the home selection goes by cells while no domain averages more home atoms
// per sort cell than this
constexpr int kCellMaxAvg = 64;

struct AGeom {
    int n[3];
    float L[3];
    float inv_c;
    float rc;
    int px;               // x index of the cell holding the cut, floor(fl(rc * inv_c))
    const float* b;       // boundaries, dimension d at boff[d]
    int boff[3];
    const int* ncell;     // cells across domain index i of d, at noff[d]
    int noff[3];
    const int* cellbase;  // first bucket of each domain
};

// Cells of a domain go row by row (row = cy + ncy * cz), along x upward in
// even rows and downward in odd ones, so the cells below the x cut at the
// end of an odd row meet those at the start of the next: the cell's key.
__device__ __forceinline__ int cell_key(const int cc[3], const int ncd[3])
{
    const int row = cc[1] + ncd[1] * cc[2];
    return ((row & 1) ? ncd[0] - 1 - cc[0] : cc[0]) + ncd[0] * row;
}

// An atom's class inside its sort cell, from the slab tests of the first
// pulses (bit d: fl(x_d - lo_d) < rc, the selection's own compare): 7 - m
// (the atoms the slabs send first) in cells whose x index differs from px by
// an even number in an even row, or by an odd one in an odd row; m (last)
// in the others. Home atoms are ordered by cell, class, global id, so a cell
// that one slab cuts keeps that pulse's atoms in one run, which meets the
// next cell's run along the row's walk.
__device__ __forceinline__ int home_class(const float u[3], const int cc[3], const int ncd[3],
                                          const AGeom& g)
{
    int m = 0;
#pragma unroll
    for (int d = 0; d < 3; d++)
        m |= (u[d] < g.rc ? 1 : 0) << d;
    const int odd = (cc[1] + ncd[1] * cc[2]) & 1;
    return (((cc[0] - g.px) ^ odd) & 1) == 0 ? 7 - m : m;
}

// Domain, sort cell and class of one position from the boundary and
// cell-count tables b and nc (laid out as in AGeom: dimension d at boff[d]
// and noff[d]); false when a coordinate lies outside [0, L) or is not a
// number. key is the cell's index inside the domain (cell_key).
__device__ __forceinline__ bool locate(const float v[3], const AGeom& g, const float* b,
                                       const int* nc, int& dom, int& key, int& cls)
{
    int ci[3], cc[3], ncd[3];
    float u[3];
#pragma unroll
    for (int d = 0; d < 3; d++) {
        if (!(v[d] >= 0.0f && v[d] < g.L[d]))
            return false;
        const float* bd = b + g.boff[d];
        const int n = g.n[d];
        int i = (int)(v[d] * ((float)n / g.L[d]));
        i = i < 0 ? 0 : (i > n - 1 ? n - 1 : i);
        while (i > 0 && v[d] < bd[i])
            i--;
        while (i < n - 1 && v[d] >= bd[i + 1])
            i++;
        ci[d] = i;
        ncd[d] = nc[g.noff[d] + i];
        u[d] = v[d] - bd[i];
        int c = 0;
        if (ncd[d] > 1) {
            const float t = u[d] * g.inv_c;
            c = (int)floorf(t);
            c = c < 0 ? 0 : (c > ncd[d] - 1 ? ncd[d] - 1 : c);
        }
        cc[d] = c;
    }
    dom = ci[0] + g.n[0] * (ci[1] + g.n[1] * ci[2]);
    key = cell_key(cc, ncd);
    cls = home_class(u, cc, ncd, g);
    return true;
}

// locate() with the boundary and cell-count tables merged per domain index:
// entry noff[d] + i of tab holds (b_d[i], b_d[i + 1], cells along d of index
// i as int bits, 0). The estimate's entry usually brackets the position, so
// one LDS read per dimension decides it (the three issued together); the
// search steps run only when it does not. Same results as locate().
__device__ __forceinline__ bool locate_tab(const float v[3], const AGeom& g, const float4* tab,
                                           int& dom, int& key, int& cls)
{
    int est[3];
    float4 e[3];
#pragma unroll
    for (int d = 0; d < 3; d++) {
        const float f = v[d] * ((float)g.n[d] / g.L[d]);
        // no conversion of NaN or of values past the last index
        int i = f >= 0.0f && f < (float)g.n[d] ? (int)f : (f >= (float)g.n[d] ? g.n[d] - 1 : 0);
        i = i > g.n[d] - 1 ? g.n[d] - 1 : i;
        est[d] = i;
        e[d] = tab[g.noff[d] + i];
    }
    int ci[3], cc[3], ncd[3];
    float u[3];
#pragma unroll
    for (int d = 0; d < 3; d++) {
        if (!(v[d] >= 0.0f && v[d] < g.L[d]))
            return false;
        const int n = g.n[d];
        int i = est[d];
        float4 t = e[d];
        if (i > 0 && v[d] < t.x) {
            do {
                i--;
                t = tab[g.noff[d] + i];
            } while (i > 0 && v[d] < t.x);
        } else if (i < n - 1 && v[d] >= t.y) {
            do {
                i++;
                t = tab[g.noff[d] + i];
            } while (i < n - 1 && v[d] >= t.y);
        }
        ci[d] = i;
        ncd[d] = __float_as_int(t.z);
        u[d] = v[d] - t.x;
        int c = 0;
        if (ncd[d] > 1) {
            c = (int)floorf(u[d] * g.inv_c);
            c = c < 0 ? 0 : (c > ncd[d] - 1 ? ncd[d] - 1 : c);
        }
        cc[d] = c;
    }
    dom = ci[0] + g.n[0] * (ci[1] + g.n[1] * ci[2]);
    key = cell_key(cc, ncd);
    cls = home_class(u, cc, ncd, g);
    return true;
}

// A home atom's sort value inside its cell: class in the top bits, global id
// below (at most 2^29 atoms), so one unsigned compare orders by class, then
// id; the per-cell sort stores the id alone.
constexpr int kClassShift = 29;
constexpr uint32_t kIdMask = (1u << kClassShift) - 1u;

// Counting form of the assignment: each atom's bucket (its domain's first
// bucket plus its cell key, -1 outside the box) and its arrival rank in the
// bucket from the count's atomic add (an arbitrary order inside the bucket,
// which the per-cell sort by class and global id then fixes), with its class
// in the rank's top bits.
__global__ __launch_bounds__(256) void assign_count_kernel(const float* __restrict__ xg,
                                                           int n_atoms, AGeom g,
                                                           int* __restrict__ bucket,
                                                           uint32_t* __restrict__ rank,
                                                           uint32_t* __restrict__ count,
                                                           uint32_t* __restrict__ err)
{
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= n_atoms)
        return;
    const float v[3] = {xg[3ll * a], xg[3ll * a + 1], xg[3ll * a + 2]};
    int dom, key, cls;
    if (!locate(v, g, g.b, g.ncell, dom, key, cls)) {
        bucket[a] = -1;
        atomicOr(err, 1u);
        return;
    }
    const int bk = g.cellbase[dom] + key;
    bucket[a] = bk;
    rank[a] = atomicAdd(count + bk, 1u) | ((uint32_t)cls << kClassShift);
}

// ---- partition sort of the home atoms (LDS counters only)

__device__ uint32_t block_scan_excl(uint32_t v, uint32_t* sh, uint32_t& total);

constexpr uint32_t kPartNone = 0xFFFFFFFFu;  // code of an atom outside the box
constexpr int kKeyBits = 12;                 // cell key bits of a code
constexpr int kDomBits = 11;                 // domain bits of a code, above the key
constexpr uint32_t kKeyMask = (1u << kKeyBits) - 1u;
constexpr uint32_t kDomMask = (1u << kDomBits) - 1u;
static_assert((1 << kKeyBits) >= kPartMaxCells, "cell keys must fit their bits");
static_assert((1 << kDomBits) >= kPartMaxDomains, "domains must fit their bits");
static_assert(kKeyBits + kDomBits + 3 < 32, "a code must differ from kPartNone");

// Partition, pass 1: tile b takes atoms [b T, (b + 1) T), T = 256 * ITEMS,
// with the geometry tables copied to LDS; stores each atom's code (class,
// domain, cell key from the top; kPartNone outside the box, reported on the
// error word) and
// counts its atoms per domain in LDS. hist[d * nblk + b] receives tile b's
// count of domain d (domain-major, so one exclusive scan gives every
// (domain, tile) its first position).
template <int ITEMS>
__global__ __launch_bounds__(256) void part_count_kernel(const float* __restrict__ xg, int n_atoms,
                                                         AGeom g, int ndom, int nblk,
                                                         uint32_t* __restrict__ code,
                                                         uint32_t* __restrict__ hist,
                                                         uint32_t* __restrict__ err)
{
    extern __shared__ float4 shq[];  // merged tables [ntab] (locate_tab), counts [ndom]
    const int ntab = g.noff[2] + g.n[2];
    float4* tab = shq;
    uint32_t* cnt = (uint32_t*)(shq + ntab);
    const int tid = (int)threadIdx.x;
    for (int d = tid; d < ndom; d += 256)
        cnt[d] = 0u;
    for (int k = tid; k < ntab; k += 256) {
        const int d = k < g.noff[1] ? 0 : (k < g.noff[2] ? 1 : 2), i = k - g.noff[d];
        const float* bd = g.b + g.boff[d];
        tab[k] = make_float4(bd[i], bd[i + 1], __int_as_float(g.ncell[k]), 0.0f);
    }
    const int blk = xcd_tile((int)blockIdx.x, (int)gridDim.x);  // neighbours share an L2
    const int64_t a0 = (int64_t)blk * (256 * ITEMS);
    // every position load of the thread is issued before the first test
    float v[ITEMS][3];
#pragma unroll
    for (int i = 0; i < ITEMS; i++) {
        const int64_t a = a0 + (int64_t)i * 256 + tid;
        const int64_t ac = a < n_atoms ? a : 0;
#pragma unroll
        for (int d = 0; d < 3; d++)
            v[i][d] = xg[3 * ac + d];
    }
    __syncthreads();
    uint32_t bad = 0u;
#pragma unroll
    for (int i = 0; i < ITEMS; i++) {
        const int64_t a = a0 + (int64_t)i * 256 + tid;
        if (a < n_atoms) {
            int dom, key, cls;
            uint32_t c = kPartNone;
            if (locate_tab(v[i], g, tab, dom, key, cls)) {
                c = ((uint32_t)cls << (kKeyBits + kDomBits)) | ((uint32_t)dom << kKeyBits) |
                    (uint32_t)key;
                atomicAdd(&cnt[dom], 1u);
            } else {
                bad = 1u;
            }
            code[a] = c;
        }
    }
    if (bad)
        atomicOr(err, 1u);
    __syncthreads();
    for (int d = tid; d < ndom; d += 256)
        hist[(int64_t)d * nblk + blk] = cnt[d];
}

// Partition, pass 2: the block's atoms grouped by domain in LDS (at an LDS
// counter's rank: any order inside a domain's share, which the per-domain
// cell sort and the per-cell sort by class and id then fix), then written out
// in that order, so each domain's share leaves as one contiguous run.
// rec[pos] gets (cell key inside the domain, class << kClassShift | global
// id) at the (domain, block)'s first position from hscan plus the rank.
template <int ITEMS>
__global__ __launch_bounds__(256) void part_scatter_kernel(const uint32_t* __restrict__ code,
                                                           int n_atoms,
                                                           const uint32_t* __restrict__ hscan,
                                                           int ndom, int nblk,
                                                           uint2* __restrict__ rec)
{
    extern __shared__ uint32_t sh[];  // staged (code, id) [(256 * ITEMS)], offset [ndom], rank [ndom]
    __shared__ uint32_t scan_sh[256];
    uint2* stage = (uint2*)sh;
    int* off = (int*)(sh + 2 * (256 * ITEMS));
    uint32_t* rnk = sh + 2 * (256 * ITEMS) + ndom;
    const int tid = (int)threadIdx.x, blk = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int64_t a0 = (int64_t)blk * (256 * ITEMS);
    uint32_t c[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; i++) {
        const int64_t a = a0 + (int64_t)i * 256 + tid;
        c[i] = a < n_atoms ? code[a] : kPartNone;
    }
    // the block's local start of each domain: a scan of its counts (each
    // thread a contiguous run of domains); off = global first - local start
    const int per = (ndom + 255) / 256;
    const int d0 = min(ndom, tid * per), d1 = min(ndom, d0 + per);
    uint32_t sum = 0u;
    for (int d = d0; d < d1; d++) {
        const int64_t h = (int64_t)d * nblk + blk;
        sum += hscan[h + 1] - hscan[h];
    }
    uint32_t total;
    uint32_t run = block_scan_excl(sum, scan_sh, total);
    for (int d = d0; d < d1; d++) {
        const int64_t h = (int64_t)d * nblk + blk;
        off[d] = (int)(hscan[h] - run);
        rnk[d] = run;
        run += hscan[h + 1] - hscan[h];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; i++) {
        if (c[i] != kPartNone) {
            const uint32_t r = atomicAdd(&rnk[(c[i] >> kKeyBits) & kDomMask], 1u);
            stage[r] = make_uint2(c[i], (uint32_t)(a0 + (int64_t)i * 256 + tid));
        }
    }
    __syncthreads();
    for (uint32_t r = tid; r < total; r += 256) {
        const uint2 e = stage[r];
        const int d = (int)((e.x >> kKeyBits) & kDomMask);
        const uint32_t cls = e.x >> (kKeyBits + kDomBits);
        rec[(int64_t)off[d] + r] = make_uint2(e.x & kKeyMask, (cls << kClassShift) | e.y);
    }
}

// Exclusive scan of v over the 1024 threads of a block (wave scans, then
// the sixteen wave totals); returns this thread's prefix.
__device__ uint32_t scan1024_excl(uint32_t v, uint32_t* wsum)
{
    const int lane = (int)threadIdx.x & 63, w = (int)threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        wsum[w] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int q = 0; q < w; q++)
        before += wsum[q];
    __syncthreads();
    return before + x - v;
}

// Order the n = e - s sort values (class << kClassShift | global id) at
// out[s, e) (one cell, ~10 atoms) and leave the global ids there: insertion
// sort in registers for up to kCellRegs values, loaded and stored once, else
// in place, then the classes cleared.
constexpr int kCellRegs = 32;
__device__ __forceinline__ void sort_cell(int* __restrict__ out, uint32_t s, uint32_t e)
{
    const int n = (int)(e - s);
    if (n <= kCellRegs) {
        uint32_t v[kCellRegs];
#pragma unroll
        for (int i = 0; i < kCellRegs; i++)
            v[i] = i < n ? (uint32_t)out[s + i] : 0xFFFFFFFFu;
        // fixed trip counts keep v[] in registers
#pragma unroll
        for (int i = 1; i < kCellRegs; i++) {
#pragma unroll
            for (int j = i; j > 0; j--) {
                const uint32_t lo = min(v[j - 1], v[j]), hi = max(v[j - 1], v[j]);
                v[j - 1] = lo;
                v[j] = hi;
            }
        }
#pragma unroll
        for (int i = 0; i < kCellRegs; i++)
            if (i < n)
                out[s + i] = (int)(v[i] & kIdMask);
        return;
    }
    for (uint32_t i = s + 1; i < e; i++) {
        const uint32_t v = (uint32_t)out[i];
        uint32_t j = i;
        while (j > s && (uint32_t)out[j - 1] > v) {
            out[j] = out[j - 1];
            j--;
        }
        out[j] = (int)v;
    }
    for (uint32_t i = s; i < e; i++)
        out[i] = (int)((uint32_t)out[i] & kIdMask);
}

// Place every sort value of rec[h0, h1) at its cell's next position in out
// (c[k] holds cell k's first position and ends as its end), then order each
// cell by class and global id, leaving the ids. out is the block's LDS copy of the domain or the domain's
// part of home_gid.
template <typename Out>
__device__ __forceinline__ void place_and_sort(const uint2* __restrict__ rec, uint32_t h0,
                                               uint32_t h1, uint32_t* c, int nc, Out* out)
{
    const int tid = (int)threadIdx.x;
    for (uint32_t i0 = h0; i0 < h1; i0 += 1024 * kDomBatch) {
        uint2 r[kDomBatch];
#pragma unroll
        for (int j = 0; j < kDomBatch; j++) {
            const uint32_t i = i0 + j * 1024 + tid;
            r[j] = i < h1 ? rec[i] : make_uint2(kPartNone, 0u);
        }
#pragma unroll
        for (int j = 0; j < kDomBatch; j++)
            if (r[j].x != kPartNone)
                out[atomicAdd(&c[r[j].x], 1u)] = (int)r[j].y;
    }
    // cell k now ends at c[k] and starts where cell k - 1 ends
    __syncthreads();
    for (int k = tid; k < nc; k += 1024)
        sort_cell(out, k ? c[k - 1] : 0u, c[k]);
}

// Positions of a sorted domain's home ranks: out[i] = xg[ids[i]] for every
// rank i whose cell the first pulses' selection by cells may read, i.e. with
// a coordinate below g.w along some dimension (cells along x, y, z in g.x,
// g.y, g.z; cell k ends at c[k]). The loads of kDomBatch ranks per thread
// are issued together.
template <typename Ids>
__device__ __forceinline__ void gather_home_positions(const Ids* ids, uint32_t n, const uint32_t* c,
                                                      int nc, const int4 g,
                                                      const float* __restrict__ xg,
                                                      float* __restrict__ out)
{
    const int tid = (int)threadIdx.x;
    const int cfx = min(g.w, g.x), cfy = min(g.w, g.y), cfz = min(g.w, g.z);
    for (uint32_t i0 = 0; i0 < n; i0 += 1024 * kDomBatch) {
        int id[kDomBatch];
#pragma unroll
        for (int j = 0; j < kDomBatch; j++) {
            const uint32_t i = i0 + j * 1024 + tid;
            id[j] = -1;
            if (i < n) {
                int lo = 0, hi = nc - 1;  // the cell k with c[k - 1] <= i < c[k]
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (c[mid] > i)
                        hi = mid;
                    else
                        lo = mid + 1;
                }
                const int row = lo / g.x, w = lo - row * g.x;  // key = w + ncx * row
                const int cx = (row & 1) ? g.x - 1 - w : w, cy = row % g.y, cz = row / g.y;
                if (cx < cfx || cy < cfy || cz < cfz)
                    id[j] = (int)ids[i];
            }
        }
        float v[kDomBatch][3];
#pragma unroll
        for (int j = 0; j < kDomBatch; j++) {
            const float* q = xg + 3ll * (id[j] < 0 ? 0 : id[j]);
            v[j][0] = q[0];
            v[j][1] = q[1];
            v[j][2] = q[2];
        }
#pragma unroll
        for (int j = 0; j < kDomBatch; j++) {
            if (id[j] >= 0) {
                float* o = out + 3ll * (i0 + j * 1024 + tid);
                o[0] = v[j][0];
                o[1] = v[j][1];
                o[2] = v[j][2];
            }
        }
    }
}

// One block per domain D, whose atoms are rec[h0, h1): count them per cell
// in LDS, scan, store the buckets' first positions (start[cellbase[D] + k],
// and start[nb] = every atom inside the box from the last domain), place
// every atom at its cell's position and order each cell by class and global
// id, then gather the home positions the selection reads into xhome. A
// domain of at most kDomCap atoms is placed and sorted in LDS and leaves in
// one coalesced copy; a larger one is placed and sorted in home_gid.
__global__ __launch_bounds__(1024) void domain_sort_kernel(const uint2* __restrict__ rec,
                                                           const uint32_t* __restrict__ hscan,
                                                           int nblk, const int* __restrict__ cellbase,
                                                           int ndom, int* __restrict__ home_gid,
                                                           uint32_t* __restrict__ start,
                                                           const float* __restrict__ xg,
                                                           const int4* __restrict__ dgeo,
                                                           float* __restrict__ xhome)
{
    __shared__ uint32_t c[kPartMaxCells];
    __shared__ int ids[kDomCap];
    __shared__ uint32_t wsum[16];
    const int D = (int)blockIdx.x, tid = (int)threadIdx.x;
    const uint32_t h0 = hscan[(int64_t)D * nblk], h1 = hscan[(int64_t)(D + 1) * nblk];
    const int cb = cellbase[D], nc = cellbase[D + 1] - cb;
    for (int k = tid; k < nc; k += 1024)
        c[k] = 0u;
    __syncthreads();
    for (uint32_t i0 = h0; i0 < h1; i0 += 1024 * kDomBatch) {
        uint32_t k[kDomBatch];
#pragma unroll
        for (int j = 0; j < kDomBatch; j++) {
            const uint32_t i = i0 + j * 1024 + tid;
            k[j] = i < h1 ? rec[i].x : kPartNone;
        }
#pragma unroll
        for (int j = 0; j < kDomBatch; j++)
            if (k[j] != kPartNone)
                atomicAdd(&c[k[j]], 1u);
    }
    __syncthreads();
    // each thread scans a contiguous run of cells
    const int per = (nc + 1023) / 1024;
    const int k0 = min(nc, tid * per), k1 = min(nc, k0 + per);
    uint32_t sum = 0;
    for (int k = k0; k < k1; k++)
        sum += c[k];
    uint32_t run = scan1024_excl(sum, wsum);
    for (int k = k0; k < k1; k++) {
        const uint32_t v = c[k];
        c[k] = run;
        start[cb + k] = h0 + run;
        run += v;
    }
    if (D == ndom - 1 && tid == 0)
        start[cellbase[ndom]] = h1;
    __syncthreads();
    const uint32_t n = h1 - h0;
    if (n <= (uint32_t)kDomCap) {
        place_and_sort(rec, h0, h1, c, nc, ids);
        __syncthreads();
        for (uint32_t i = tid; i < n; i += 1024)
            home_gid[h0 + i] = ids[i];
        gather_home_positions(ids, n, c, nc, dgeo[D], xg, xhome + 3ll * h0);
    } else {
        place_and_sort(rec, h0, h1, c, nc, home_gid + h0);
        // this block's stores to home_gid are visible to its own threads
        // after the barrier
        __syncthreads();
        gather_home_positions(home_gid + h0, n, c, nc, dgeo[D], xg, xhome + 3ll * h0);
    }
}

// ---- exclusive scan of uint32 counts: out[i] = sum(in[0..i)), out[n] = total

__device__ uint32_t block_scan_excl(uint32_t v, uint32_t* sh, uint32_t& total)
{
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const uint32_t add = t >= o ? sh[t - o] : 0u;
        __syncthreads();
        sh[t] += add;
        __syncthreads();
    }
    total = sh[255];
    const uint32_t incl = sh[t];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(256) void scan_sums_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                        uint32_t* __restrict__ bsum)
{
    __shared__ uint32_t sh[256];
    const int64_t b0 = (int64_t)blockIdx.x * kScanBlock + 4ll * threadIdx.x;
    uint32_t s = 0;
    for (int k = 0; k < 4; k++)
        if (b0 + k < n)
            s += in[b0 + k];
    uint32_t total;
    block_scan_excl(s, sh, total);
    if (threadIdx.x == 0)
        bsum[blockIdx.x] = total;
}

// Second pass: each block first sums the totals of the blocks before it
// (strided loads, then wavefront shuffles), then scans its own elements;
// the last block also stores the grand total at out[n].
__global__ __launch_bounds__(256) void scan_apply_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                         const uint32_t* __restrict__ bsum,
                                                         uint32_t* __restrict__ out)
{
    __shared__ uint32_t sh[256];
    __shared__ uint32_t wred[4];
    uint32_t part = 0;
    for (int i = (int)threadIdx.x; i < (int)blockIdx.x; i += 256)
        part += bsum[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        part += __shfl_down(part, o, 64);
    if ((threadIdx.x & 63) == 0)
        wred[threadIdx.x >> 6] = part;
    __syncthreads();
    const uint32_t pre = wred[0] + wred[1] + wred[2] + wred[3];
    const int64_t b0 = (int64_t)blockIdx.x * kScanBlock + 4ll * threadIdx.x;
    uint32_t v[4];
    uint32_t s = 0;
    for (int k = 0; k < 4; k++) {
        v[k] = b0 + k < n ? in[b0 + k] : 0u;
        s += v[k];
    }
    uint32_t total;
    uint32_t run = pre + block_scan_excl(s, sh, total);
    for (int k = 0; k < 4; k++) {
        if (b0 + k < n)
            out[b0 + k] = run;
        run += v[k];
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0)
        out[n] = pre + total;
}

// Every atom's sort value (class << kClassShift | global id) to its bucket's
// range, at its arrival rank (an arbitrary order inside the bucket: the
// per-cell sort by class and global id fixes it).
__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ bucket,
                                                      const uint32_t* __restrict__ rank,
                                                      int n_atoms,
                                                      const uint32_t* __restrict__ start,
                                                      int* __restrict__ sorted)
{
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= n_atoms)
        return;
    const int bk = bucket[a];
    if (bk < 0)
        return;  // a position outside the box: reported by the build
    const uint32_t r = rank[a];
    sorted[start[bk] + (r & kIdMask)] = (int)((r & ~kIdMask) | (uint32_t)a);
}

// Order each cell's atoms by class and global id (one thread per cell).
__global__ __launch_bounds__(256) void sort_cells_kernel(const uint32_t* __restrict__ start, int nb,
                                                         int* __restrict__ sorted)
{
    const int bk = blockIdx.x * 256 + threadIdx.x;
    if (bk < nb)
        sort_cell(sorted, start[bk], start[bk + 1]);
}

__global__ void home_start_kernel(const uint32_t* __restrict__ start, const int* __restrict__ cellbase,
                                  int ndom, int* __restrict__ hs)
{
    const int D = blockIdx.x * 256 + threadIdx.x;
    if (D <= ndom)
        hs[D] = (int)start[cellbase[D]];
}

// ---- per-pulse selection

struct STile;  // one slot tile of a pulse's selection (below)

struct SArgs {
    int d;
    float L_d, rc;
    const STile* tiles;   // [b] selection tile b
    const float* lo;      // per S: lower boundary along d
    const int* shiftbit;  // per S: 1 if S sits at index 0 of d
    const int* map_pos;   // per S: first entry of its map in the pulse buffer
    int* map_out;
    const int* out_pos;   // per S: first record of its region at R
    int* out_gid;
    float* out_xyz;
    // the pulse's entries (pulse_totals_kernel) and the room of map_out,
    // out_gid and out_xyz: the write does nothing when they do not fit
    const uint32_t* total;
    uint32_t cap;
    // The pulse's counting units, sender-major: sender S's candidate home
    // cells (with the selection by cells, CArgs; hcprefix null otherwise),
    // then its tiles, at ubase[S] on; one exclusive scan of the units' counts
    // gives each its first entry.
    const int* ubase;
    const int* hcprefix;
};

// Units of sender S before its tiles (its candidate home cells).
__device__ __forceinline__ int home_units(const SArgs& a, int S)
{
    return a.hcprefix ? a.hcprefix[S + 1] - a.hcprefix[S] : 0;
}

// slot_gid and home_slot of the home atoms: work item b (of ndom * cpd,
// grid-strided) fills chunk b % cpd (kFillTile home ranks) of domain b /
// cpd, whose ranks [hs[D], hs[D + 1]) take slots from base[D] on.
constexpr int kFillItems = 8;
constexpr int kFillTile = 256 * kFillItems;
constexpr int kFillMaxBlocks = 1 << 20;
__global__ __launch_bounds__(256) void fill_home_kernel(const int* __restrict__ home_gid,
                                                        const int* __restrict__ hs,
                                                        const int* __restrict__ base, int ndom,
                                                        int cpd, int* __restrict__ slot_gid,
                                                        int* __restrict__ home_slot,
                                                        uint8_t* __restrict__ rid)
{
    for (int64_t b = blockIdx.x; b < (int64_t)ndom * cpd; b += gridDim.x) {
        const int D = (int)(b / cpd), c = (int)(b % cpd);
        const int64_t r0 = hs[D] + (int64_t)c * kFillTile;
        const int64_t r1 = min((int64_t)hs[D + 1], r0 + kFillTile);
        if (r0 >= r1)
            continue;
        const int64_t off = (int64_t)base[D] - hs[D];
        int g[kFillItems];
#pragma unroll
        for (int j = 0; j < kFillItems; j++) {
            const int64_t r = r0 + j * 256 + (int)threadIdx.x;
            g[j] = r < r1 ? home_gid[r] : 0;
        }
#pragma unroll
        for (int j = 0; j < kFillItems; j++) {
            const int64_t r = r0 + j * 256 + (int)threadIdx.x;
            if (r < r1) {
                slot_gid[r + off] = g[j];
                home_slot[r] = (int)(r + off);
                rid[r + off] = 0xff;
            }
        }
    }
}

// Slab selection of pulse p in tiles (the slab test of the pulse's dimension
// d: fl(x_d - lo_d(S)) < rc): each tile of the pulse (tiles of S numbered
// from tprefix[S], in slot order) is one block. Counting and writing by tile
// fills the GPU whatever the number of domains; an exclusive scan of the
// tile counts (in S order, then slot order) gives every tile its first entry
// in the pulse's map buffer, so the compaction stays in slot order.
//
// One slot tile of a pulse's selection: sender S's candidate slots
// [j0, j1), all from one source (its home slots, home = 1, or the records
// one earlier pulse delivered to it), whose global ids and positions (float3,
// the periodic shift of the delivering pulse already applied: the value the
// coordinate pass leaves in the slot) start at gid and xyz for slot j0. The
// host cuts each sender's candidate range at its sources' bounds and then
// into tiles of at most kSelTile slots, so a block reads its tile's source
// once instead of resolving every slot.
struct STile {
    const int* gid;
    const float* xyz;
    int S, j0, j1, home;
};

// ---- slab selection of the home slots by cells (a dimension's first pulse)
//
// A home atom's cell coordinate along d is floor(fl(u * inv_c)), clamped to
// the domain's cells, of the same u = fl(x_d - lo_d(S)) that the slab test
// fl(x_d - lo_d(S)) < rc compares, and fl(u * inv_c) is monotone in u. So
// from the host's thresholds, a sender's cells with coordinate >= cfail
// along d hold only failing positions and are never visited, and those
// below cpass hold only passing ones and are taken whole without reading a
// position. Only the cells in between are tested atom by atom. The
// candidate cells of a sender are numbered m = 0, 1, ... in key order (=
// slot order); the count takes one thread per cell, the write one thread
// per slot of 256 consecutive cells.
struct CArgs {
    int d;
    float L_d, rc;
    const int* ctile_s;    // [b] sender of cell tile b (256 candidate cells)
    const int* ctprefix;   // [S] first cell tile of S
    const int* hcprefix;   // [S] first candidate cell of S in the pulse's numbering
    const int4* cls;       // [S] cells along x, along y, certain-pass and candidate cells along d
    const int* cellbase;   // first bucket of each domain
    const uint32_t* start; // home rank where each bucket starts
    const int* home_start;
    const float* xhome;
    const int* home_gid;
    const float* lo;
    const int* shiftbit;
    int nblocks;           // cell tiles (the launch's first blocks)
    const int* map_pos;
    int* map_out;
    const int* out_pos;
    int* out_gid;
    float* out_xyz;
};

// Candidate cell m of a sender: its key (cell_key) and its coordinate along
// d. Along z the candidates are the layers cz < cf, along y the rows cy < cf
// of every layer, along x the cells cx < cf of every row: the first cf keys
// of an even row and the last cf, cx descending, of an odd one.
__device__ __forceinline__ int cand_cell(int m, int d, int ncx, int ncy, int cf, int& cd)
{
    if (d == 2) {
        cd = m / (ncx * ncy);
        return m;
    }
    if (d == 1) {
        const int per = ncx * cf, cz = m / per, r = m - cz * per;
        cd = r / ncx;
        return r + cz * ncx * ncy;
    }
    const int row = m / cf, i = m - row * cf;
    if (row & 1) {
        cd = cf - 1 - i;
        return ncx - cf + i + ncx * row;
    }
    cd = i;
    return i + ncx * row;
}

constexpr int kCellBatch = 16;  // positions of a cell a thread loads together

// The home ranks [r0, r1) of candidate cell m of cell tile cb's sender and
// whether they pass whole; false when m is past the sender's candidates.
__device__ __forceinline__ bool cand_range(const CArgs& a, int cb, int& S, int& m, uint32_t& r0,
                                           uint32_t& r1, bool& whole)
{
    S = a.ctile_s[cb];
    m = (cb - a.ctprefix[S]) * 256 + (int)threadIdx.x;
    if (m >= a.hcprefix[S + 1] - a.hcprefix[S])
        return false;
    const int4 k = a.cls[S];
    int cd;
    const int key = cand_cell(m, a.d, k.x, k.y, k.w, cd);
    const int bk = a.cellbase[S] + key;
    r0 = a.start[bk];
    r1 = a.start[bk + 1];
    whole = cd < k.z;
    return true;
}

// Count of cell tile cb: each candidate cell's entries, at its unit.
__device__ void cell_count_block(const CArgs& a, int cb, const int* ubase, uint32_t* ucnt)
{
    int S, m;
    uint32_t r0, r1;
    bool whole;
    if (!cand_range(a, cb, S, m, r0, r1, whole))
        return;
    uint32_t n = r1 - r0;
    if (!whole) {
        const float lo = a.lo[S];
        n = 0;
        for (uint32_t b = r0; b < r1; b += kCellBatch) {
            float v[kCellBatch];
#pragma unroll
            for (int i = 0; i < kCellBatch; i++)
                v[i] = b + i < r1 ? a.xhome[3ll * (b + i) + a.d] : __builtin_nanf("");
#pragma unroll
            for (int i = 0; i < kCellBatch; i++)
                n += (v[i] - lo) < a.rc;  // false for NaN
        }
    }
    ucnt[ubase[S] + m] = n;
}

// Write of cell tile cb: its candidate cells (256 consecutive ones of one sender) as one
// run of home slots: each thread loads its cell's range into LDS, a block
// scan lays the cells end to end, and the block walks that run 256 slots
// at a time. Every slot of a whole cell is selected, every other one is
// tested; a ballot prefix over the block gives each selected slot its entry,
// so consecutive lanes read consecutive slots and write consecutive entries.
__device__ void cell_write_block(const CArgs& a, int cb, const int* ubase, const uint32_t* uscan)
{
    __shared__ uint32_t cr0[256];
    __shared__ int cst[257];
    __shared__ unsigned char cwhole[256];
    __shared__ uint32_t scan_sh[256];
    __shared__ int wt[4];
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int S = a.ctile_s[cb];
    const int m0 = (cb - a.ctprefix[S]) * 256;
    const int ncb = min(256, a.hcprefix[S + 1] - a.hcprefix[S] - m0);  // cells of the block
    uint32_t r0 = 0, r1 = 0;
    bool whole = false;
    if (tid < ncb) {
        const int4 k = a.cls[S];
        int cd;
        const int key = cand_cell(m0 + tid, a.d, k.x, k.y, k.w, cd);
        const int bk = a.cellbase[S] + key;
        r0 = a.start[bk];
        r1 = a.start[bk + 1];
        whole = cd < k.z;
    }
    uint32_t nslots;
    const uint32_t off = block_scan_excl(r1 - r0, scan_sh, nslots);
    cr0[tid] = r0;
    cst[tid] = (int)off;
    cwhole[tid] = whole;
    if (tid == 0)
        cst[ncb] = (int)nslots;
    __syncthreads();
    const float lo = a.lo[S];
    const int hs = a.home_start[S];
    const bool shift = a.shiftbit[S] != 0;
    // the block's first entry: S's entries of the cells before the block
    int run = (int)(uscan[ubase[S] + m0] - uscan[ubase[S]]);
    int* map = a.map_out + a.map_pos[S];
    int* gid = a.out_gid + a.out_pos[S];
    float* xyz = a.out_xyz + 3ll * a.out_pos[S];
    for (int base = 0; base < (int)nslots; base += 256) {
        const int t = base + tid;
        bool pass = false;
        uint32_t r = 0;
        float v0 = 0.0f, v1 = 0.0f, v2 = 0.0f;
        int g = 0;
        if (t < (int)nslots) {
            int l = 0, h = ncb;  // the cell c with cst[c] <= t < cst[c + 1]
            while (h - l > 1) {
                const int mid = (l + h) >> 1;
                if (cst[mid] <= t)
                    l = mid;
                else
                    h = mid;
            }
            r = cr0[l] + (uint32_t)(t - cst[l]);
            v0 = a.xhome[3ll * r];
            v1 = a.xhome[3ll * r + 1];
            v2 = a.xhome[3ll * r + 2];
            g = a.home_gid[r];
            const float vd = a.d == 0 ? v0 : a.d == 1 ? v1 : v2;
            pass = cwhole[l] || (vd - lo) < a.rc;
        }
        const unsigned long long bal = __ballot(pass);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0)
            wt[w] = __popcll(bal);
        __syncthreads();
        int before = 0, tot = 0;
        for (int q = 0; q < 4; q++) {
            before += q < w ? wt[q] : 0;
            tot += wt[q];
        }
        if (pass) {
            const int idx = run + before + pre;
            map[idx] = (int)r - hs;
            gid[idx] = g;
            // the record as the receiver gets it: + L_d on component d when
            // the sender sits at index 0 of d
            xyz[3ll * idx] = (a.d == 0 && shift) ? v0 + a.L_d : v0;
            xyz[3ll * idx + 1] = (a.d == 1 && shift) ? v1 + a.L_d : v1;
            xyz[3ll * idx + 2] = (a.d == 2 && shift) ? v2 + a.L_d : v2;
        }
        run += tot;
        __syncthreads();  // wt is rewritten next round
    }
}

// Counts of the pulse's units: the first ca.nblocks blocks are cell tiles
// (cell_count_block), the others slot tiles, each counting its selected
// slots and those below the split (home slots).
__global__ __launch_bounds__(256) void select_count_kernel(SArgs a, CArgs ca,
                                                           const int* __restrict__ tprefix,
                                                           uint32_t* __restrict__ ucnt,
                                                           uint32_t* __restrict__ below)
{
    if ((int)blockIdx.x < ca.nblocks) {
        cell_count_block(ca, (int)blockIdx.x, a.ubase, ucnt);
        return;
    }
    const int tb = (int)blockIdx.x - ca.nblocks;
    __shared__ int s_send;
    const STile t = a.tiles[tb];
    const int S = t.S, n = t.j1 - t.j0;
    if (threadIdx.x == 0)
        s_send = 0;
    __syncthreads();
    int c = 0;
    const float lo = a.lo[S];
    // the tile's kSelTile / 256 slots per thread: every position load is
    // issued before the first test, so the loads are in flight together
    constexpr int U = kSelTile / 256;
    float v[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int i = (int)threadIdx.x + u * 256;
        v[u] = i < n ? t.xyz[3ll * i + a.d] : __builtin_nanf("");
    }
#pragma unroll
    for (int u = 0; u < U; u++)
        c += (v[u] - lo) < a.rc;  // false for the NaN of a slot out of range
    atomicAdd(&s_send, c);
    __syncthreads();
    if (threadIdx.x == 0) {
        ucnt[a.ubase[S] + home_units(a, S) + (tb - tprefix[S])] = (uint32_t)s_send;
        below[tb] = t.home ? (uint32_t)s_send : 0u;
    }
}

// Per-sender totals of a pulse from the unit scan: entries sent (cnt_send)
// and entries below the split (home slots: cnt_split). Then the write
// offsets: map_pos[S], S's first entry in the pulse's maps (exclusive prefix
// over senders); out_pos[S], the first record of S's region in the pulse's
// received storage (exclusive prefix of the region sizes in receiver order:
// S sends to rcv[S], R receives from snd[R]; rstart holds the prefix per
// receiver); and the pulse's total. One block of 1024 threads.
__global__ __launch_bounds__(1024) void pulse_totals_kernel(SArgs a, const int* __restrict__ tprefix,
                                                            int ndom,
                                                            const uint32_t* __restrict__ scan,
                                                            const uint32_t* __restrict__ below,
                                                            int* __restrict__ cnt_send,
                                                            int* __restrict__ cnt_split,
                                                            const int* __restrict__ rcv,
                                                            const int* __restrict__ snd,
                                                            int* __restrict__ map_pos,
                                                            int* __restrict__ rstart,
                                                            int* __restrict__ out_pos,
                                                            uint32_t* __restrict__ total)
{
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t s_tot;
    const int tid = (int)threadIdx.x;
    uint32_t carry = 0;
    for (int b = 0; b < ndom; b += 1024) {
        const int S = b + tid;
        uint32_t cs = 0;
        if (S < ndom) {
            const int u0 = a.ubase[S];
            cs = scan[a.ubase[S + 1]] - scan[u0];
            uint32_t bl = scan[u0 + home_units(a, S)] - scan[u0];  // home cells: all below
            for (int t = tprefix[S]; t < tprefix[S + 1]; t++)
                bl += below[t];
            cnt_send[S] = (int)cs;
            cnt_split[S] = (int)bl;
        }
        const uint32_t e = scan1024_excl(cs, wsum);
        if (S < ndom)
            map_pos[S] = (int)(carry + e);
        if (tid == 1023)
            s_tot = e + cs;
        __syncthreads();
        carry += s_tot;
        __syncthreads();
    }
    if (tid == 0)
        *total = carry;
    // (the barriers above order the cnt_send stores for the whole block)
    carry = 0;
    for (int b = 0; b < ndom; b += 1024) {
        const int R = b + tid;
        const uint32_t v = R < ndom ? (uint32_t)cnt_send[snd[R]] : 0u;
        const uint32_t e = scan1024_excl(v, wsum);
        if (R < ndom)
            rstart[R] = (int)(carry + e);
        if (tid == 1023)
            s_tot = e + v;
        __syncthreads();
        carry += s_tot;
        __syncthreads();
    }
    for (int S = tid; S < ndom; S += 1024)
        out_pos[S] = rstart[rcv[S]];
}

// Ordered compaction of one tile: its selected slots go to the sender's map
// from the tile's scanned offset on, in slot order.
__global__ __launch_bounds__(256) void select_write_kernel(SArgs a, CArgs ca,
                                                           const int* __restrict__ tprefix,
                                                           const uint32_t* __restrict__ scan)
{
    if (*a.total > a.cap)  // the same for every block: the host grows the room and repeats
        return;
    if ((int)blockIdx.x < ca.nblocks) {
        cell_write_block(ca, (int)blockIdx.x, a.ubase, scan);
        return;
    }
    const int tb = (int)blockIdx.x - ca.nblocks;
    __shared__ int wave_tot[4];
    __shared__ int s_run;
    const STile t = a.tiles[tb];
    const int S = t.S, n = t.j1 - t.j0;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0)  // S's entries of the units before this tile
        s_run = (int)(scan[a.ubase[S] + home_units(a, S) + (tb - tprefix[S])] - scan[a.ubase[S]]);
    __syncthreads();
    const bool shift = a.shiftbit[S] != 0;
    const float lo = a.lo[S];
    // as in the count: every slot's position load is issued before the
    // first test
    constexpr int U = kSelTile / 256;
    float v[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int i = (int)threadIdx.x + u * 256;
        v[u] = i < n ? t.xyz[3ll * i + a.d] : __builtin_nanf("");
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int i = (int)threadIdx.x + u * 256;
        const int j = t.j0 + i;
        const bool pred = (v[u] - lo) < a.rc;  // false for the NaN of a slot out of range
        const unsigned long long bal = __ballot(pred);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0)
            wave_tot[w] = __popcll(bal);
        __syncthreads();
        int off = s_run, tot = 0;
        for (int q = 0; q < 4; q++) {
            if (q < w)
                off += wave_tot[q];
            tot += wave_tot[q];
        }
        if (pred) {
            const int idx = off + pre;
            a.map_out[a.map_pos[S] + idx] = j;
            a.out_gid[a.out_pos[S] + idx] = t.gid[i];
            // the record as the receiver gets it: + L_d on component d when
            // the sender sits at index 0 of d
            const float* pos = t.xyz + 3ll * i;
            float* o = a.out_xyz + 3ll * (a.out_pos[S] + idx);
            for (int c = 0; c < 3; c++) {
                float r = pos[c];
                if (c == a.d && shift)
                    r = r + a.L_d;
                o[c] = r;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0)
            s_run += tot;
        __syncthreads();
    }
}

// Segmented work for the per-record kernels below: nseg segments, segment
// k holding items [pre[k], pre[k + 1]). Work item b (of nseg * cps, grid-
// strided) is chunk b % cps (kSegTile items) of segment b / cps, so a block
// knows its segment without searching for it. Returns false when the chunk
// is empty.
constexpr int kSegItems = 8;
constexpr int kSegTile = 256 * kSegItems;
constexpr int kSegMaxBlocks = 1 << 20;
__device__ __forceinline__ bool seg_chunk(const int* pre, int cps, int64_t b, int& k, int& i0,
                                          int& i1)
{
    k = (int)(b / cps);
    const int c = (int)(b % cps);
    i0 = pre[k] + c * kSegTile;
    i1 = min(pre[k + 1], i0 + kSegTile);
    return i0 < i1;
}

// Region q of every receiver: global id of each received slot, and the pulse
// it was received in (rid). Receiver R's records are rs[R] .. rs[R + 1] of
// the pulse's storage and land at slots dst[R] on.
__global__ __launch_bounds__(256) void fill_region_kernel(const int* __restrict__ rgid,
                                                          const int* __restrict__ rs, int ndom,
                                                          int cps, const int* __restrict__ dst,
                                                          int* __restrict__ slot_gid,
                                                          uint8_t* __restrict__ rid, int q)
{
    for (int64_t b = blockIdx.x; b < (int64_t)ndom * cps; b += gridDim.x) {
        int R, i0, i1;
        if (!seg_chunk(rs, cps, b, R, i0, i1))
            continue;
        const int off = dst[R] - rs[R];
        int g[kSegItems];
#pragma unroll
        for (int j = 0; j < kSegItems; j++) {
            const int i = i0 + j * 256 + (int)threadIdx.x;
            g[j] = i < i1 ? rgid[i] : 0;
        }
#pragma unroll
        for (int j = 0; j < kSegItems; j++) {
            const int i = i0 + j * 256 + (int)threadIdx.x;
            if (i < i1) {
                slot_gid[i + off] = g[j];
                rid[i + off] = (uint8_t)q;
            }
        }
    }
}

// The pulses' maps (written by the selection, one buffer per pulse) joined
// pulse-major into one array: entry i of pulse q lands at begin[q] + i, in
// 32 bits and, when out16 is given (every domain has at most 65536 slots, so
// every sender-local index fits), in 16 bits as well.
struct MapParts {
    const int32_t* src[DDH_MAX_PULSES];
    int64_t begin[DDH_MAX_PULSES + 1];
    int P;
};

__global__ __launch_bounds__(256) void join_maps_kernel(MapParts mp, int32_t* __restrict__ out,
                                                        uint16_t* __restrict__ out16)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int q = 0; q < mp.P; q++) {  // uniform: the pulse's table entries stay scalar
        const int32_t* src = mp.src[q];
        const int64_t b0 = mp.begin[q], n = mp.begin[q + 1] - b0;
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
            const int32_t v = src[i];
            out[b0 + i] = v;
            if (out16)
                out16[b0 + i] = (uint16_t)v;
        }
    }
}

// Home positions in slot order: xhome[r] = xg[home_gid[r]] (float3).
__global__ __launch_bounds__(256) void gather_xhome_kernel(const float* __restrict__ xg,
                                                           const int* __restrict__ home_gid,
                                                           int n, float* __restrict__ xhome)
{
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= n)
        return;
    const float* src = xg + 3ll * home_gid[r];
    float* dst = xhome + 3ll * r;
    dst[0] = src[0];
    dst[1] = src[1];
    dst[2] = src[2];
}

// Per-map data of a build for the device-made chunk tables: [S * P + q].
struct MapInfo {
    const int* send;     // map size
    const int* recv;     // receiver
    const int* roff;     // the region's first slot at the receiver
    const int* map_off;  // first entry in the map array
    const int* shift;    // 1 if the sender sits at index 0 of the pulse's dimension
    const int* base;     // [domain] first slot
    const int* pdim;     // [pulse] dimension
    float L[3];
    int D, P;
};

// The per-pulse launches' chunk table (no waits): chunk k of a map of n
// entries in c chunks is the slice [n k / c, n (k + 1) / c). Coordinate
// chunks are listed pulse by pulse, sender by sender (xprefix: first chunk
// of each (pulse, sender) unit, in that order); force chunks in decreasing
// pulse order (fprefix). One thread per chunk.
__global__ __launch_bounds__(256) void pulse_chunks_kernel(MapInfo m, const int* __restrict__ nchunks,
                                                           const int* __restrict__ xprefix, int nx,
                                                           const int* __restrict__ fprefix, int nf,
                                                           DChunk* __restrict__ xch,
                                                           DChunk* __restrict__ fch)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= nx + nf)
        return;
    const bool force = c >= nx;
    const int cc = force ? c - nx : c;
    const int* pre = force ? fprefix : xprefix;
    int lo = 0, hi = m.D * m.P;  // the unit u with pre[u] <= cc < pre[u + 1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= cc)
            lo = mid;
        else
            hi = mid;
    }
    const int r = lo / m.D, S = lo - r * m.D;
    const int q = force ? m.P - 1 - r : r;
    const int it = S * m.P + q, k = cc - pre[lo];
    const int n = m.send[it], nc = nchunks[it];
    DChunk d{};
    d.hb = (int32_t)((int64_t)n * k / nc);
    d.he = (int32_t)((int64_t)n * (k + 1) / nc);
    d.tb = d.te = d.he;
    d.src_base = m.base[S];
    d.R = m.recv[it];
    d.dst_base = m.base[d.R] + m.roff[it];
    d.map_off = m.map_off[it];
    const int dim = m.pdim[q];
    d.flags = dim | (m.shift[it] ? kChunkShift : 0);
    d.shift = m.L[dim];
    d.S = S;
    d.p = q;
    d.ctr = force ? S * m.P + q : d.R * m.P + q;
    (force ? fch : xch)[cc] = d;
}

// Chunk-aligned copy of the maps for the per-pulse launches: block b writes
// the entries of chunk b at out[b * CH ...] and zeros up to the next chunk;
// block 0 also clears the kPadTail entries after the last chunk.
template <typename T>
__global__ __launch_bounds__(256) void pad_maps_kernel(const T* __restrict__ maps,
                                                       const DChunk* __restrict__ ch, int CH,
                                                       T* __restrict__ out)
{
    const DChunk c = ch[blockIdx.x];
    const int n = c.he - c.hb;
    T* o = out + (int64_t)blockIdx.x * CH;
    for (int i = threadIdx.x; i < CH; i += 256)
        o[i] = i < n ? maps[c.map_off + c.hb + i] : (T)0;
    if (blockIdx.x == 0) {
        T* tail = out + (int64_t)gridDim.x * CH;
        for (int i = threadIdx.x; i < kPadTail; i += 256)
            tail[i] = (T)0;
    }
}

// inmap[slot] |= bit for every entry of pulse q's maps (maps_q: the pulse's
// maps of all senders, sender S's at mpos[S]..mpos[S+1], segmented as in
// fill_region_kernel). Within one pulse every slot appears at most once (a
// map holds distinct slots of its own sender), so plain read-modify-writes
// suffice; pulses run one after the other on the stream.
__global__ __launch_bounds__(256) void inmap_kernel(const int32_t* __restrict__ maps_q,
                                                    const int* __restrict__ mpos, int ndom, int cps,
                                                    const int* __restrict__ base,
                                                    uint32_t* __restrict__ inmap, uint32_t bit)
{
    for (int64_t b = blockIdx.x; b < (int64_t)ndom * cps; b += gridDim.x) {
        int S, i0, i1;
        if (!seg_chunk(mpos, cps, b, S, i0, i1))
            continue;
        int slot[kSegItems];
#pragma unroll
        for (int j = 0; j < kSegItems; j++) {
            const int i = i0 + j * 256 + (int)threadIdx.x;
            slot[j] = i < i1 ? base[S] + maps_q[i] : -1;
        }
#pragma unroll
        for (int j = 0; j < kSegItems; j++)
            if (slot[j] >= 0)
                inmap[slot[j]] |= bit;
    }
}

// Wait masks of the fused launch's chunks, one block per chunk. Coordinate
// chunk: the pulses whose regions at S its dependent slice reads (bit
// rid[slot] of every entry of [tb, te)). Force chunk: the later pulses whose
// maps hold a slot it adds into (at S) or a slot of R's region it reads.
__global__ __launch_bounds__(256) void chunk_masks_kernel(DChunk* __restrict__ xch, int nx,
                                                          DChunk* __restrict__ fch, int nf,
                                                          const int32_t* __restrict__ maps,
                                                          const uint8_t* __restrict__ rid,
                                                          const uint32_t* __restrict__ inmap,
                                                          int P)
{
    __shared__ uint32_t s_a, s_b;
    if (threadIdx.x == 0) {
        s_a = 0u;
        s_b = 0u;
    }
    __syncthreads();
    const int b = (int)blockIdx.x;
    uint32_t wa = 0u, wb = 0u;
    if (b < nx) {
        const DChunk c = xch[b];
        for (int i = c.tb + (int)threadIdx.x; i < c.te; i += 256) {
            const uint8_t r = rid[c.src_base + maps[c.map_off + i]];
            if (r < 32)
                wa |= 1u << r;
        }
    } else {
        const DChunk c = fch[b - nx];
        for (int i = c.hb + (int)threadIdx.x; i < c.he; i += 256) {
            wa |= inmap[c.src_base + maps[c.map_off + i]];
            wb |= inmap[c.dst_base + i];
        }
    }
    if (wa)
        atomicOr(&s_a, wa);
    if (wb)
        atomicOr(&s_b, wb);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (b < nx) {
            xch[b].wait_a = s_a;
        } else {
            DChunk& c = fch[b - nx];
            const uint32_t later = ~((2u << c.p) - 1u) & ((1u << P) - 1u);
            c.wait_a = s_a & later;
            c.wait_b = s_b & later;
        }
    }
}

// ---------------------------------------------------------------- host side

// Device buffers used only during a build. They stay with the plan between
// builds (maps are rebuilt every neighbour-search step): the k-th request of
// a build reuses the k-th buffer of the previous one when it is large
// enough, and grows it otherwise. A build waits for its stream before it
// returns, so no work of an earlier build still uses them; after a failed
// build the next one first waits for the device.
struct Scratch {
    Plan* plan;
    size_t next = 0;
    size_t pnext = 0;
    explicit Scratch(Plan* p) : plan(p) {}
    // Pinned host staging for one upload: slot k serves the k-th upload of
    // every build and is reused while large enough (a build's uploads have
    // all run by its final sync, before the next build reuses a slot). From
    // pinned memory hipMemcpyAsync returns at once; from pageable memory the
    // host would first wait for the stream, leaving the device idle while
    // it prepares the next work.
    hipError_t pinned(void** out, size_t n)
    {
        const size_t bytes = (std::max<size_t>(n, 1) + 255) & ~size_t(255);
        auto& cache = plan->pinned;
        if (pnext < cache.size() && cache[pnext].second >= bytes) {
            *out = cache[pnext++].first;
            return hipSuccess;
        }
        void* q = nullptr;
        hipError_t e = hipHostMalloc(&q, bytes, hipHostMallocDefault);
        if (e != hipSuccess) {
            *out = nullptr;
            return e;
        }
        if (pnext < cache.size()) {
            (void)hipHostFree(cache[pnext].first);
            cache[pnext] = {q, bytes};
        } else {
            cache.emplace_back(q, bytes);
        }
        pnext++;
        *out = q;
        return hipSuccess;
    }
    // An asynchronous upload of n bytes through a pinned staging slot.
    hipError_t upload_bytes(void* dst, const void* src, size_t n, hipStream_t s)
    {
        if (n == 0)
            return hipSuccess;
        void* h;
        const hipError_t e = pinned(&h, n);
        if (e != hipSuccess)
            return e;
        std::memcpy(h, src, n);
        return hipMemcpyAsync(dst, h, n, hipMemcpyHostToDevice, s);
    }
    template <class T>
    hipError_t alloc(T** out, size_t n)
    {
        const size_t bytes = (std::max<size_t>(n, 1) * sizeof(T) + 255) & ~size_t(255);
        auto& cache = plan->scratch;
        if (next < cache.size() && cache[next].second >= bytes) {
            *out = (T*)cache[next++].first;
            return hipSuccess;
        }
        void* q = nullptr;
        hipError_t e = hipMalloc(&q, bytes);
        if (e != hipSuccess) {
            *out = nullptr;
            return e;
        }
        if (next < cache.size()) {
            (void)hipFree(cache[next].first);
            cache[next] = {q, bytes};
        } else {
            cache.emplace_back(q, bytes);
        }
        next++;
        *out = (T*)q;
        return hipSuccess;
    }
};

// Device memory of the built state. Slot k of the plan's kept list serves the
// k-th allocation of every build and is reused while it is large enough, so a
// rebuild (every neighbour-search step) allocates nothing once sizes settle.
// The plan frees the list when it is destroyed.
template <class T>
hipError_t owned_alloc(Plan* p, T** out, size_t n)
{
    const size_t bytes = (std::max<size_t>(n, 1) * sizeof(T) + 255) & ~size_t(255);
    auto& kept = p->kept;
    const size_t k = p->kept_next++;
    if (k < kept.size() && kept[k].second >= bytes) {
        *out = (T*)kept[k].first;
        return hipSuccess;
    }
    void* q = nullptr;
    hipError_t e = hipMalloc(&q, bytes);
    if (e != hipSuccess) {
        *out = nullptr;
        return e;
    }
    if (k < kept.size()) {
        (void)hipFree(kept[k].first);
        kept[k] = {q, bytes};
    } else {
        kept.emplace_back(q, bytes);
    }
    *out = (T*)q;
    return hipSuccess;
}

// Small host arrays gathered into one host-to-device copy: add() appends a
// section (16-byte aligned) and returns its byte offset; send() copies the
// whole blob into a scratch buffer (staged through pinned memory, so the
// blob itself may go out of scope at once), after which section k sits at
// base + offset k.
struct Blob {
    std::vector<uint64_t> words;
    size_t bytes = 0;
    template <class T>
    size_t add(const T* src, size_t n)
    {
        const size_t off = (bytes + 15) & ~size_t(15);
        bytes = off + n * sizeof(T);
        words.resize((bytes + 7) / 8);
        if (n)
            std::memcpy(reinterpret_cast<char*>(words.data()) + off, src, n * sizeof(T));
        return off;
    }
    template <class T>
    size_t add(const std::vector<T>& v)
    {
        return add(v.data(), v.size());
    }
    hipError_t send(Scratch& sc, char** base, hipStream_t s)
    {
        hipError_t e = sc.alloc(base, std::max<size_t>(bytes, 8));
        if (e != hipSuccess || bytes == 0)
            return e;
        return sc.upload_bytes(*base, words.data(), bytes, s);
    }
};

template <class T>
hipError_t upload(Scratch& sc, T* dst, const std::vector<T>& src, hipStream_t s)
{
    return sc.upload_bytes(dst, src.data(), src.size() * sizeof(T), s);
}

int scan_exclusive(Scratch& sc, const uint32_t* in, int64_t n, uint32_t* out, hipStream_t s)
{
    const int nblk = (int)((n + kScanBlock - 1) / kScanBlock);
    uint32_t* bsum;
    DDH_HIP(sc.alloc(&bsum, (size_t)nblk + 1));
    if (nblk > 0)
        hipLaunchKernelGGL(scan_sums_kernel, dim3(nblk), dim3(256), 0, s, in, n, bsum);
    // (one block when n is 0: it stores the total, 0)
    hipLaunchKernelGGL(scan_apply_kernel, dim3(std::max(nblk, 1)), dim3(256), 0, s, in, n, bsum,
                       out);
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

int blocks(int64_t n) { return (int)((n + 255) / 256); }

}  // namespace

void free_scratch(Plan* p)
{
    for (auto& kv : p->scratch)
        (void)hipFree(kv.first);
    p->scratch.clear();
    for (auto& kv : p->pinned)
        (void)hipHostFree(kv.first);
    p->pinned.clear();
    for (auto& kv : p->kept)
        (void)hipFree(kv.first);
    p->kept.clear();
    p->kept_next = 0;
    for (auto& kv : p->selbuf)
        (void)hipFree(kv.first);
    p->selbuf.clear();
    if (p->counts_ready)
        (void)hipEventDestroy(p->counts_ready);
    p->counts_ready = nullptr;
}

void free_built(Plan* p)
{
    for (auto& kv : p->graphs)
        (void)hipGraphExecDestroy(kv.second);
    p->graphs.clear();
    for (void* q : p->owned)
        (void)hipFree(q);
    p->owned.clear();
    p->kept_next = 0;
    p->d_maps = p->d_slot_gid = p->d_home_gid = p->d_home_slot = nullptr;
    p->d_maps16 = nullptr;
    p->d_rid = nullptr;
    p->fused_ready = false;
    p->fused = WorkTable{};
    p->pulse = WorkTable{};
    p->pulse1 = WorkTable{};
    p->d_ctrl = p->d_xcnt = p->d_fcnt = p->d_xneed = p->d_fneed = p->d_pflag = nullptr;
    p->d_stage = nullptr;
    p->built = false;
    p->n_slots = p->n_halo = 0;
    p->n_atoms = 0;
}

// Chunk table of chunk size t.chunk. With waits (the fused launch) a
// coordinate chunk takes the k-th slice of its map's independent head and of
// its dependent tail (with wavefront workers: the k-th contiguous slice of
// the map, whose entries at or past the split form its tail), and a force
// chunk the k-th slice of the map; the wait masks are the conservative ones
// (every earlier / later pulse) unless refined waits are on, in which case
// chunk_masks_kernel fills them in from the maps. Without waits (per-pulse
// launches, ordered by the stream) every chunk is one contiguous slice and
// the masks stay empty.
static void make_work_table(const Plan* p, bool waits, WorkTable& t)
{
    const Geometry& g = p->g;
    const int D = g.ndom, P = g.P, CH = t.chunk;
    t.nchunks.assign((size_t)D * P, 1);
    for (int it = 0; it < D * P; it++)
        t.nchunks[it] = std::max(1, (p->send[it] + CH - 1) / CH);

    auto base_chunk = [&](int it) {
        const int S = it / P, q = it % P;
        DChunk d{};
        d.src_base = (int32_t)p->base[S];
        d.R = p->recv[it];
        d.dst_base = (int32_t)(p->base[d.R] + p->roff[it]);
        d.map_off = (int32_t)p->map_off[it];
        d.flags = g.pdim[q] | (p->shift[it] ? kChunkShift : 0);
        d.shift = g.L[g.pdim[q]];
        d.S = S;
        d.p = q;
        return d;
    };
    const bool conservative = waits && !p->fused_refined;  // as set at the build
    // coordinates: the k-th slice of the independent head and of the
    // dependent tail; the chunk advances the counter of the region it fills
    auto xchunk = [&](int it, int k) {
        const int c = t.nchunks[it], h = p->split[it], tl = p->send[it] - h;
        DChunk d = base_chunk(it);
        d.ctr = d.R * P + d.p;
        if (!waits) {
            const int n = p->send[it];
            d.hb = (int32_t)((int64_t)n * k / c);
            d.he = (int32_t)((int64_t)n * (k + 1) / c);
            d.tb = d.te = d.he;
            return d;
        }
        if (t.wave) {
            const int n = p->send[it];
            const int b = (int)((int64_t)n * k / c), e = (int)((int64_t)n * (k + 1) / c);
            d.hb = b;
            d.he = std::max(b, std::min(e, h));
            d.tb = std::min(std::max(b, h), e);
            d.te = e;
        } else {
            d.hb = (int32_t)((int64_t)h * k / c);
            d.he = (int32_t)((int64_t)h * (k + 1) / c);
            d.tb = h + (int32_t)((int64_t)tl * k / c);
            d.te = h + (int32_t)((int64_t)tl * (k + 1) / c);
        }
        d.wait_a = (conservative && d.te > d.tb) ? (1u << d.p) - 1u : 0u;
        return d;
    };
    // forces: the k-th slice of the map; the chunk advances its own item's
    // counter
    auto fchunk = [&](int it, int k) {
        const int c = t.nchunks[it], n = p->send[it];
        DChunk d = base_chunk(it);
        d.hb = (int32_t)((int64_t)n * k / c);
        d.he = (int32_t)((int64_t)n * (k + 1) / c);
        d.tb = d.te = d.he;
        d.ctr = d.S * P + d.p;
        const uint32_t later = ~((2u << d.p) - 1u) & ((1u << P) - 1u);
        d.wait_a = d.wait_b = conservative ? later : 0u;
        return d;
    };

    t.xch.clear();
    t.fch.clear();
    t.xpulse_begin.assign((size_t)P + 1, 0);
    t.fpulse_begin.assign((size_t)P + 1, 0);
    if (waits && t.heads_first && !t.wave) {
        // heads first: every map's independent head in chunks of its own,
        // all of them (pulse order) before any dependent tail (pulse
        // order), so no head ever waits and the tails follow the regions
        // they read. A map has ceil(h / CH) head and ceil(tl / CH) tail
        // chunks (an empty map one empty head chunk), and the force pass
        // slices it into the same number of chunks. xpulse_begin marks the
        // heads of each pulse only (the fused launch does not use it).
        std::vector<int> nh((size_t)D * P), nt((size_t)D * P);
        for (int it = 0; it < D * P; it++) {
            const int h = p->split[it], tl = p->send[it] - h;
            nh[it] = (h + CH - 1) / CH;
            nt[it] = (tl + CH - 1) / CH;
            if (nh[it] + nt[it] == 0)
                nh[it] = 1;
            t.nchunks[it] = nh[it] + nt[it];
        }
        for (int q = 0; q < P; q++) {
            t.xpulse_begin[q] = (int)t.xch.size();
            for (int S = 0; S < D; S++) {
                const int it = S * P + q, h = p->split[it];
                for (int k = 0; k < nh[it]; k++) {
                    DChunk d = base_chunk(it);
                    d.ctr = d.R * P + d.p;
                    d.hb = (int32_t)((int64_t)h * k / nh[it]);
                    d.he = (int32_t)((int64_t)h * (k + 1) / nh[it]);
                    d.tb = d.te = d.he;
                    t.xch.push_back(d);
                }
            }
        }
        for (int q = 0; q < P; q++)
            for (int S = 0; S < D; S++) {
                const int it = S * P + q, h = p->split[it], tl = p->send[it] - h;
                for (int k = 0; k < nt[it]; k++) {
                    DChunk d = base_chunk(it);
                    d.ctr = d.R * P + d.p;
                    d.hb = d.he = h;
                    d.tb = h + (int32_t)((int64_t)tl * k / nt[it]);
                    d.te = h + (int32_t)((int64_t)tl * (k + 1) / nt[it]);
                    d.wait_a = conservative ? (1u << d.p) - 1u : 0u;
                    t.xch.push_back(d);
                }
            }
    } else {
        // coordinates in pulse order (a chunk waits only on earlier pulses)
        for (int q = 0; q < P; q++) {
            t.xpulse_begin[q] = (int)t.xch.size();
            for (int S = 0; S < D; S++)
                for (int k = 0; k < t.nchunks[S * P + q]; k++)
                    t.xch.push_back(xchunk(S * P + q, k));
        }
    }
    t.xpulse_begin[P] = (int)t.xch.size();
    t.nx = (int)t.xch.size();
    // forces in decreasing pulse order (a chunk waits only on later pulses)
    for (int r = 0; r < P; r++) {
        const int q = P - 1 - r;
        t.fpulse_begin[r] = (int)t.fch.size();
        for (int S = 0; S < D; S++)
            for (int k = 0; k < t.nchunks[S * P + q]; k++)
                t.fch.push_back(fchunk(S * P + q, k));
    }
    t.fpulse_begin[P] = (int)t.fch.size();
    t.nf = (int)t.fch.size();
}

// Device form of set_release_flags (below), for masks computed on the
// device: read[S * P + q] marks a coordinate counter, read[DP + S * P + q] a
// force counter that some chunk waits on (every writer stores 1).
__global__ __launch_bounds__(256) void release_marks_kernel(const DChunk* __restrict__ xch, int nx,
                                                            const DChunk* __restrict__ fch, int nf,
                                                            int P, int DP,
                                                            uint32_t* __restrict__ read)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < nx) {
        const DChunk& c = xch[i];
        for (uint32_t m = c.wait_a; m; m &= m - 1)
            read[c.S * P + __builtin_ctz(m)] = 1u;
    } else if (i < nx + nf) {
        const DChunk& c = fch[i - nx];
        for (uint32_t m = c.wait_a; m; m &= m - 1)
            read[DP + c.S * P + __builtin_ctz(m)] = 1u;
        for (uint32_t m = c.wait_b; m; m &= m - 1)
            read[DP + c.R * P + __builtin_ctz(m)] = 1u;
    }
}

__global__ __launch_bounds__(256) void release_apply_kernel(DChunk* __restrict__ xch, int nx,
                                                            DChunk* __restrict__ fch, int nf, int DP,
                                                            const uint32_t* __restrict__ read)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < nx) {
        if (read[xch[i].ctr])
            xch[i].flags |= kChunkRelease;
    } else if (i < nx + nf) {
        if (read[DP + fch[i - nx].ctr])
            fch[i - nx].flags |= kChunkRelease;
    }
}

// A chunk of the fused launch publishes with a release fence only if a
// later chunk of the same launch waits on its counter (and so reads what it
// wrote). Needs the final wait masks.
static void set_release_flags(const Plan* p, WorkTable& t)
{
    const int D = p->g.ndom, P = p->g.P;
    std::vector<char> xread((size_t)D * P, 0), fread((size_t)D * P, 0);
    for (const DChunk& c : t.xch)
        for (uint32_t m = c.wait_a; m; m &= m - 1)
            xread[(size_t)c.S * P + __builtin_ctz(m)] = 1;
    for (const DChunk& c : t.fch) {
        for (uint32_t m = c.wait_a; m; m &= m - 1)
            fread[(size_t)c.S * P + __builtin_ctz(m)] = 1;
        for (uint32_t m = c.wait_b; m; m &= m - 1)
            fread[(size_t)c.R * P + __builtin_ctz(m)] = 1;
    }
    for (DChunk& c : t.xch)
        if (xread[c.ctr])
            c.flags |= kChunkRelease;
    for (DChunk& c : t.fch)
        if (fread[c.ctr])
            c.flags |= kChunkRelease;
}

// Entries per chunk of the fused launch: 8192, which gives one chunk per map
// on every workload measured, each run by one 1024-wide work-group. That
// keeps the device-wide serialized operations (ticket claims, releases,
// acquires) few: 12M atoms 316 -> 222 us per fused step against 4096, 1M
// 42.0 -> 37.5 us. With wavefront workers: 1024 (16 entries per lane;
// smaller slices multiply the serialized ticket claims and releases).
static int fused_chunk(const Plan* p) { return p->wave_chunks ? 1024 : 8192; }

// Entries per chunk of the per-pulse launches (256-lane blocks, up to eight
// entries per lane and round), from the average entries of a pulse per
// compute unit, a. Measured on MI355X (graph replay, us per step; each pass
// alone in brackets):
//   - a >= 4096 (12M atoms on 8x8x8 domains, a = 11000): 2048, for steps
//     (111.0; 1024: 118.0, 1536: 114.7, 2560: 117.8, 3072: 115.4) and, since
//     neighbouring chunks are dealt to one XCD, for a pass alone too (one
//     table for both: coordinates 48.3 against 48.9 at 1024, forces 68.1
//     against 68.9);
//   - a >= 256 (1M atoms on 4x4x4, a = 1080; 384k atoms on 16x4x4, a = 1050):
//     768 (1M: 17.15, 512: 17.15, 1024: 17.44; 384k: 22.85, 1024: 22.82, 512:
//     23.46, the former one chunk per map of up to 2752 entries: 27.4);
//   - smaller (96k atoms on 2x2x2, a = 93): 256 (8.95; 128: 9.32, 512: 9.18).
// But first, for the table of step calls, where some chunk size of at most
// 4096 entries keeps every launch at one chunk per compute unit or fewer,
// the smallest such multiple of 256: a launch then takes as long as its
// largest chunk (maps are split into equal parts). 1M: 2816 (16.1 us per
// step; 768: 17.1; 2560, whose launch of the Z coordinates and X forces has
// 320 chunks: 19.9; 3584, which leaves maps of 3499 entries whole: 18.5).
// 12M and 384k have more maps than compute units per launch and keep the
// rule below. Single-pass launches carry half the work and keep it too
// (the same rule for them: 1M coordinates 10.9 -> 11.4 us at 1536, 384k
// 15.7 -> 16.2 at 2816).
// step: the table of step calls (both passes share each launch), else the
// one of single-pass calls.
static int pulse_chunk(const Plan* p, bool step)
{
    const int P = p->g.P, D = p->g.ndom;
    const int ncu = std::max(1, p->n_cu);
    auto chunks = [&](int q, int ch) {  // chunks of pulse q's maps (one at least each)
        int64_t c = 0;
        for (int S = 0; S < D; S++)
            c += std::max(1, (p->send[(size_t)S * P + q] + ch - 1) / ch);
        return c;
    };
    for (int ch = kSmallChunk; step && ch <= 4096 && P > 0; ch += 256) {
        int64_t most = 0;  // chunks of the table's largest launch
        for (int q = 0; q < P; q++)
            most = std::max(most, chunks(q, ch) + chunks(P - 1 - q, ch));
        if (most <= ncu)
            return ch;
    }
    int64_t total = 0;
    for (int32_t n : p->send)
        total += n;
    const int64_t a = P > 0 ? total / P / ncu : 0;
    if (a >= 4096)
        return 2048;
    if (a >= 256)
        return 768;
    return kSmallChunk;
}

// A per-pulse launches' table of chunk size t.chunk, made on the device.
// Host part: each map's chunk count and the table's pulse ranges; returns
// the first chunk of every (pulse, sender) unit, coordinates then forces.
static std::vector<int> pulse_table_counts(const Plan* p, WorkTable& t)
{
    const int D = p->g.ndom, P = p->g.P, CH = t.chunk;
    t.wave = false;
    t.heads_first = false;
    t.xch.clear();
    t.fch.clear();
    t.nchunks.assign((size_t)D * P, 1);
    for (int it = 0; it < D * P; it++)
        t.nchunks[it] = std::max(1, (p->send[it] + CH - 1) / CH);
    // first chunk of each unit: coordinates (pulse, sender), then forces
    // (reverse pulse, sender)
    std::vector<int> pre(2 * ((size_t)D * P + 1), 0);
    int* xpre = pre.data();
    int* fpre = pre.data() + (size_t)D * P + 1;
    t.xpulse_begin.assign((size_t)P + 1, 0);
    t.fpulse_begin.assign((size_t)P + 1, 0);
    for (int r = 0; r < P; r++) {
        t.xpulse_begin[r] = xpre[r * D];
        t.fpulse_begin[r] = fpre[r * D];
        for (int S = 0; S < D; S++) {
            const int u = r * D + S;
            xpre[u + 1] = xpre[u] + t.nchunks[S * P + r];
            fpre[u + 1] = fpre[u] + t.nchunks[S * P + (P - 1 - r)];
        }
    }
    t.nx = xpre[D * P];
    t.nf = fpre[D * P];
    t.xpulse_begin[P] = t.nx;
    t.fpulse_begin[P] = t.nf;
    return pre;
}

// Device part (d_pre, d_nch: the host part's output on the device): the
// descriptors (pulse_chunks_kernel), then the chunk-aligned copies of the
// maps (coordinate chunk k's entries at slot k * chunk, force chunks sharing
// the slot of the coordinate chunk of the same map slice).
static int make_pulse_table(Plan* p, const MapInfo& m, WorkTable& t, const int* d_pre,
                            const int* d_nch, hipStream_t s)
{
    const int D = p->g.ndom, P = p->g.P;
    DDH_HIP(owned_alloc(p, &t.d_xch, (size_t)t.nx));
    DDH_HIP(owned_alloc(p, &t.d_fch, (size_t)t.nf));
    if (t.nx + t.nf > 0)
        hipLaunchKernelGGL(pulse_chunks_kernel, dim3(blocks(t.nx + t.nf)), dim3(256), 0, s, m, d_nch,
                           d_pre, t.nx, d_pre + (size_t)D * P + 1, t.nf, t.d_xch, t.d_fch);
    DDH_HIP(hipGetLastError());
    // the copy kernel writes every chunk's slot (entries, then zeros) and
    // the tail after the last one (no chunk: nothing reads the copy). The
    // 32-bit copy is made only
    // when the 16-bit maps are off (without it, launches read the maps
    // after the descriptor).
    const int nch = t.nx;
    const size_t body = (size_t)nch * t.chunk, npad = body + kPadTail;
    t.d_pad = nullptr;
    t.d_pad16 = nullptr;
    if (!p->d_maps16 || !p->narrow_maps) {
        DDH_HIP(owned_alloc(p, &t.d_pad, npad));
        if (nch > 0)
            hipLaunchKernelGGL(pad_maps_kernel<int32_t>, dim3(nch), dim3(256), 0, s, p->d_maps,
                               t.d_xch, t.chunk, t.d_pad);
    }
    if (p->d_maps16) {
        DDH_HIP(owned_alloc(p, &t.d_pad16, npad));
        if (nch > 0)
            hipLaunchKernelGGL(pad_maps_kernel<uint16_t>, dim3(nch), dim3(256), 0, s, p->d_maps16,
                               t.d_xch, t.chunk, t.d_pad16);
    }
    DDH_HIP(hipGetLastError());
    return DDH_OK;
}

// Consecutive named host ranges for the phases of one build.
struct Phases {
    bool open = false;
    void next(const char* name)
    {
        if (open)
            roctxRangePop();
        roctxRangePushA(name);
        open = true;
    }
    ~Phases()
    {
        if (open)
            roctxRangePop();
    }
};

// The fused launch's chunk table (chunk size, wavefront workers, heads
// first and refined waits as set at the build), its wait masks and release
// flags (on the device from the maps, with refined waits), and the counter
// target of every map. Needs the build's maps, slot bases, slot pulses and
// counters.
static int fused_stage(Plan* p, Scratch& sc, hipStream_t s)
{
    const int D = p->g.ndom, P = p->g.P;
    const size_t DP = (size_t)D * P;
    WorkTable& t = p->fused;
    make_work_table(p, true, t);
    DDH_HIP(owned_alloc(p, &t.d_xch, t.xch.size()));
    DDH_HIP(owned_alloc(p, &t.d_fch, t.fch.size()));
    if (p->fused_refined && P > 0) {
        DDH_HIP(upload(sc, t.d_xch, t.xch, s));
        DDH_HIP(upload(sc, t.d_fch, t.fch, s));
        // per pulse: each sender's first entry in the pulse's maps, then
        // the pulse's total; the slot bases
        std::vector<int> mposall(((size_t)D + 1) * P);
        int64_t pb = 0;
        for (int q = 0; q < P; q++) {
            int64_t tot = 0;
            for (int S = 0; S < D; S++) {
                mposall[(size_t)q * (D + 1) + S] = (int)(p->map_off[(size_t)S * P + q] - pb);
                tot += p->send[(size_t)S * P + q];
            }
            mposall[(size_t)q * (D + 1) + D] = (int)tot;
            pb += tot;
        }
        std::vector<int> base32(D);
        for (int Dm = 0; Dm < D; Dm++)
            base32[Dm] = (int)p->base[Dm];
        Blob mb;
        const size_t o_mpos = mb.add(mposall), o_base = mb.add(base32);
        char* d_mb;
        DDH_HIP(mb.send(sc, &d_mb, s));
        const int* d_mpos = (const int*)(d_mb + o_mpos);
        const int* d_base = (const int*)(d_mb + o_base);
        uint32_t* d_inmap;
        DDH_HIP(sc.alloc(&d_inmap, (size_t)p->n_slots));
        DDH_HIP(hipMemsetAsync(d_inmap, 0, sizeof(uint32_t) * (size_t)p->n_slots, s));
        pb = 0;
        for (int q = 0; q < P; q++) {
            const int total = mposall[(size_t)q * (D + 1) + D];
            int max_map = 0;  // the largest map of the pulse, in chunks
            for (int S = 0; S < D; S++)
                max_map = std::max(max_map, p->send[(size_t)S * P + q]);
            const int cps = (max_map + kSegTile - 1) / kSegTile;
            if (total > 0 && cps > 0)
                hipLaunchKernelGGL(inmap_kernel,
                                   dim3((unsigned)std::min<int64_t>((int64_t)D * cps, kSegMaxBlocks)),
                                   dim3(256), 0, s, p->d_maps + pb, d_mpos + (size_t)q * (D + 1), D,
                                   cps, d_base, d_inmap, 1u << q);
            pb += total;
        }
        const int nx = (int)t.xch.size(), nf = (int)t.fch.size();
        // the release flags follow from the masks, on the device as well
        // (the host copies of the fused table keep neither)
        uint32_t* d_read;
        DDH_HIP(sc.alloc(&d_read, 2 * DP));
        DDH_HIP(hipMemsetAsync(d_read, 0, sizeof(uint32_t) * 2 * DP, s));
        if (nx + nf > 0) {
            hipLaunchKernelGGL(chunk_masks_kernel, dim3(nx + nf), dim3(256), 0, s, t.d_xch, nx,
                               t.d_fch, nf, p->d_maps, p->d_rid, d_inmap, P);
            hipLaunchKernelGGL(release_marks_kernel, dim3(blocks(nx + nf)), dim3(256), 0, s,
                               t.d_xch, nx, t.d_fch, nf, P, (int)DP, d_read);
            hipLaunchKernelGGL(release_apply_kernel, dim3(blocks(nx + nf)), dim3(256), 0, s,
                               t.d_xch, nx, t.d_fch, nf, (int)DP, d_read);
        }
        DDH_HIP(hipGetLastError());
    } else {
        set_release_flags(p, t);
        DDH_HIP(upload(sc, t.d_xch, t.xch, s));
        DDH_HIP(upload(sc, t.d_fch, t.fch, s));
    }
    // counter targets: chunks per map (coordinates at the receiver's row)
    std::vector<uint32_t> need(2 * DP, 0u);
    for (int S = 0; S < D; S++)
        for (int q = 0; q < P; q++) {
            const size_t it = (size_t)S * P + q;
            need[(size_t)p->recv[it] * P + q] = (uint32_t)t.nchunks[it];
            need[DP + it] = (uint32_t)t.nchunks[it];
        }
    // d_fneed follows d_xneed: one copy of both
    DDH_HIP(upload(sc, p->d_xneed, need, s));
    return DDH_OK;
}

int build_maps(Plan* p, const float* xg, int32_t n_atoms, hipStream_t s)
{
    Phases ph;
    free_built(p);
    Geometry& g = p->g;
    const int D = g.ndom, P = g.P;
    if (n_atoms < 0 || (n_atoms > 0 && !xg))
        return fail(DDH_EINVAL, "ddh_build_maps: bad positions pointer or count");
    if ((int64_t)n_atoms > (int64_t)kIdMask + 1)
        return fail(DDH_EINVAL, "ddh_build_maps: at most 2^29 atoms");
    if (p->build_failed)
        DDH_HIP(hipDeviceSynchronize());  // kernels of the failed build may still run
    p->build_failed = true;
    Scratch sc(p);

    // ---- geometry tables
    ph.next("build: geometry");
    std::vector<float> bcat;
    std::vector<int> ncat;
    AGeom ag{};
    for (int d = 0; d < 3; d++) {
        ag.n[d] = g.n[d];
        ag.L[d] = g.L[d];
        ag.boff[d] = (int)bcat.size();
        ag.noff[d] = (int)ncat.size();
        bcat.insert(bcat.end(), g.b[d].begin(), g.b[d].end());
        ncat.insert(ncat.end(), g.ncell[d].begin(), g.ncell[d].end());
    }
    ag.inv_c = g.inv_c;
    ag.rc = g.rc;
    ag.px = (int)std::floor(g.rc * g.inv_c);
    std::vector<int> cellbase((size_t)D + 1, 0);
    {
        int64_t acc = 0;
        for (int Dm = 0; Dm < D; Dm++) {
            int c[3];
            g.coords(Dm, c);
            cellbase[Dm] = (int)acc;
            acc += (int64_t)g.ncell[0][c[0]] * g.ncell[1][c[1]] * g.ncell[2][c[2]];
            if (acc > (1ll << 30))
                return fail(DDH_EINVAL, "ddh_build_maps: too many sort cells (cell edge too small)");
        }
        cellbase[D] = (int)acc;
    }
    const int nb = cellbase[D];
    // Cell thresholds of the home selection (cell_count_block): umin(c) is
    // the smallest u >= 0 whose cell coordinate floor(fl(u * inv_c))
    // reaches c. Along d, cell c holds only passing positions when
    // umin(c + 1) <= rc (and it is not the domain's last cell, which also
    // takes every larger u), only failing ones when umin(c) >= rc.
    int cpass0 = 0, cfail0 = 1;
    if (g.inv_c > 0.0f) {
        auto umin = [&](int c) {
            uint32_t lo = 0u, hi = 0x7F800000u;  // +inf reaches every c
            while (lo < hi) {
                const uint32_t mid = lo + (hi - lo) / 2;
                float u;
                std::memcpy(&u, &mid, 4);
                if (u * g.inv_c >= (float)c)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            float u;
            std::memcpy(&u, &lo, 4);
            return u;
        };
        while (cpass0 < (1 << 20) && umin(cpass0 + 1) <= g.rc)
            cpass0++;
        while (cfail0 < (1 << 20) && umin(cfail0) < g.rc)
            cfail0++;
    }
    // per domain: cells along x, y, z, and the first cell index along any
    // dimension that no first pulse's selection reads (cfail0: the home sort
    // gathers only the positions of the other cells; a huge value gathers all)
    std::vector<int> dgeo(4 * (size_t)D);
    for (int Dm = 0; Dm < D; Dm++) {
        int c[3];
        g.coords(Dm, c);
        dgeo[4 * Dm] = g.ncell[0][c[0]];
        dgeo[4 * Dm + 1] = g.ncell[1][c[1]];
        dgeo[4 * Dm + 2] = g.ncell[2][c[2]];
        dgeo[4 * Dm + 3] = g.inv_c > 0.0f ? cfail0 : INT32_MAX;
    }
    Blob geo;
    const size_t o_b = geo.add(bcat), o_ncell = geo.add(ncat), o_cellbase = geo.add(cellbase);
    const size_t o_dgeo = geo.add(dgeo);
    // the home starts, then the error word (zero): read back in one copy
    const std::vector<int> hs0((size_t)D + 2, 0);
    const size_t o_hs = geo.add(hs0);
    char* d_geo;
    DDH_HIP(geo.send(sc, &d_geo, s));
    int* d_hs = (int*)(d_geo + o_hs);
    uint32_t* d_err = (uint32_t*)(d_hs + D + 1);
    const int* d_cellbase = (const int*)(d_geo + o_cellbase);
    const int4* d_dgeo = (const int4*)(d_geo + o_dgeo);
    ag.b = (const float*)(d_geo + o_b);
    ag.ncell = (const int*)(d_geo + o_ncell);
    ag.cellbase = d_cellbase;

    // ---- 1-2: home assignment and cell sort
    ph.next("build: assign and sort");
    // Two forms, same order. Partition (the default wherever its LDS tables
    // fit): block histograms of the atoms per domain in LDS, one scan, a
    // scatter into per-domain segments with LDS counters, then one block per
    // domain counting its atoms per cell in LDS and placing them; no device
    // atomic on any atom. Counting (any size): a device atomic count per
    // bucket gives each atom its arrival rank, a scan the bucket starts, a
    // scatter the positions. Both then sort each cell by class and global id.
    int max_cells = 0;
    for (int Dm = 0; Dm < D; Dm++)
        max_cells = std::max(max_cells, cellbase[Dm + 1] - cellbase[Dm]);
    const bool fits = D <= kPartMaxDomains && max_cells <= kPartMaxCells;
    const bool partition = p->home_sort == 2 ? true : (p->home_sort == 0 && fits);
    if (partition && !fits)
        return fail(DDH_EINVAL, "ddh_build_maps: the partition sort (DDH_TUNE_HOME_SORT 2) needs "
                                "at most 2048 domains and 4096 sort cells per domain");
    uint32_t* d_start;
    DDH_HIP(sc.alloc(&d_start, (size_t)nb + 1));
    DDH_HIP(owned_alloc(p, &p->d_home_gid, (size_t)n_atoms));
    // home positions in slot order: the slab tests read them in order
    float* d_xhome;
    DDH_HIP(sc.alloc(&d_xhome, 3 * (size_t)n_atoms));
    if (partition) {
        const int items = (int64_t)n_atoms >= 16ll * 256 * kPartMinBlocks ? 16
                          : (int64_t)n_atoms >= 4ll * 256 * kPartMinBlocks ? 4 : 1;
        const int tile = 256 * items;
        const int nblk = (int)(((int64_t)n_atoms + tile - 1) / tile);
        const size_t part_lds = sizeof(float4) * (size_t)(ag.noff[2] + ag.n[2]) + sizeof(uint32_t) * D;
        uint32_t *d_code, *d_hist, *d_hscan;
        uint2* d_rec;
        DDH_HIP(sc.alloc(&d_code, (size_t)n_atoms));
        DDH_HIP(sc.alloc(&d_hist, (size_t)D * nblk + 1));
        DDH_HIP(sc.alloc(&d_hscan, (size_t)D * nblk + 1));
        DDH_HIP(sc.alloc(&d_rec, (size_t)n_atoms));
        const auto count_k = items == 16 ? part_count_kernel<16>
                             : items == 4 ? part_count_kernel<4> : part_count_kernel<1>;
        const auto scatter_k = items == 16 ? part_scatter_kernel<16>
                               : items == 4 ? part_scatter_kernel<4> : part_scatter_kernel<1>;
        if (nblk > 0)
            hipLaunchKernelGGL(count_k, dim3(nblk), dim3(256), part_lds, s, xg, n_atoms, ag, D, nblk,
                               d_code, d_hist, d_err);
        DDH_HIP(hipGetLastError());
        // (domain, block) first positions; hscan[D * nblk] = atoms in the box
        const int rc = scan_exclusive(sc, d_hist, (int64_t)D * nblk, d_hscan, s);
        if (rc)
            return rc;
        if (nblk > 0)
            hipLaunchKernelGGL(scatter_k, dim3(nblk), dim3(256),
                               sizeof(uint32_t) * (2 * (size_t)tile + 2 * (size_t)D), s, d_code,
                               n_atoms, d_hscan, D, nblk, d_rec);
        hipLaunchKernelGGL(domain_sort_kernel, dim3(D), dim3(1024), 0, s, d_rec, d_hscan, nblk,
                           d_cellbase, D, p->d_home_gid, d_start, xg, d_dgeo, d_xhome);
        DDH_HIP(hipGetLastError());
    } else {
        int* d_bucket;
        uint32_t *d_count, *d_rank;
        DDH_HIP(sc.alloc(&d_bucket, (size_t)n_atoms));
        DDH_HIP(sc.alloc(&d_rank, (size_t)n_atoms));
        DDH_HIP(sc.alloc(&d_count, (size_t)nb + 1));
        DDH_HIP(hipMemsetAsync(d_count, 0, sizeof(uint32_t) * ((size_t)nb + 1), s));
        if (n_atoms > 0)
            hipLaunchKernelGGL(assign_count_kernel, dim3(blocks(n_atoms)), dim3(256), 0, s, xg,
                               n_atoms, ag, d_bucket, d_rank, d_count, d_err);
        DDH_HIP(hipGetLastError());
        // atoms outside the box have no bucket and are skipped until the
        // error word is read with the home counts below
        const int rc = scan_exclusive(sc, d_count, nb, d_start, s);
        if (rc)
            return rc;
        if (n_atoms > 0) {
            hipLaunchKernelGGL(scatter_kernel, dim3(blocks(n_atoms)), dim3(256), 0, s, d_bucket,
                               d_rank, n_atoms, d_start, p->d_home_gid);
            hipLaunchKernelGGL(sort_cells_kernel, dim3(blocks(nb)), dim3(256), 0, s, d_start, nb,
                               p->d_home_gid);
        }
    }
    hipLaunchKernelGGL(home_start_kernel, dim3(blocks(D + 1)), dim3(256), 0, s, d_start, d_cellbase,
                       D, d_hs);
    DDH_HIP(hipGetLastError());
    // the home starts and the error word, read back through pinned memory
    // (both copies queued, one wait)
    std::vector<int> hs((size_t)D + 1);
    uint32_t herr = 0;
    {
        void* h;
        DDH_HIP(sc.pinned(&h, sizeof(int) * ((size_t)D + 2)));
        int* hp = (int*)h;
        DDH_HIP(hipMemcpyAsync(hp, d_hs, sizeof(int) * (D + 2), hipMemcpyDeviceToHost, s));
        DDH_HIP(hipStreamSynchronize(s));
        std::memcpy(hs.data(), hp, sizeof(int) * ((size_t)D + 1));
        std::memcpy(&herr, hp + D + 1, sizeof(uint32_t));
    }
    if (herr)
        return fail(DDH_EINVAL, "ddh_build_maps: a position is outside [0, L) or not a number");
    p->nhome.assign(D, 0);
    p->ntotal.assign(D, 0);
    for (int Dm = 0; Dm < D; Dm++) {
        p->nhome[Dm] = hs[Dm + 1] - hs[Dm];
        p->ntotal[Dm] = p->nhome[Dm];
    }
    // the first pulses select home slots by cells while cells are small (a
    // thread walks each candidate cell)
    bool cell_mode = g.inv_c > 0.0f;
    for (int Dm = 0; Dm < D && cell_mode; Dm++)
        cell_mode = p->nhome[Dm] <= (int64_t)kCellMaxAvg * (cellbase[Dm + 1] - cellbase[Dm]);
    // the partition sort gathered the positions the selection by cells
    // reads; otherwise every home position is gathered here
    if (n_atoms > 0 && (!partition || (!cell_mode && g.inv_c > 0.0f)))
        hipLaunchKernelGGL(gather_xhome_kernel, dim3(blocks(n_atoms)), dim3(256), 0, s, xg,
                           p->d_home_gid, n_atoms, d_xhome);
    DDH_HIP(hipGetLastError());

    // ---- 3: pulses
    ph.next("build: pulses");
    const size_t DP = (size_t)D * P;
    p->send.assign(DP, 0);
    p->split.assign(DP, 0);
    p->recv.assign(DP, 0);
    p->roff.assign(DP, 0);
    p->shift.assign(DP, 0);
    std::vector<int> roff_at(DP, 0), rsize_at(DP, 0), rstart(DP, 0);
    std::vector<int*> rgid((size_t)std::max(P, 1), nullptr);
    std::vector<float*> rxyz((size_t)std::max(P, 1), nullptr);
    std::vector<int*> mapp((size_t)std::max(P, 1), nullptr);
    std::vector<std::vector<int>> mpos((size_t)P), rsprefix((size_t)P);
    std::vector<int> total((size_t)P, 0);
    int *d_cnt_send, *d_cnt_split;  // adjacent: read back in one copy
    DDH_HIP(sc.alloc(&d_cnt_send, 2 * (size_t)D));
    d_cnt_split = d_cnt_send + D;

    // the pulses' upload blobs
    std::vector<Blob> blobs;
    blobs.reserve(2 * (size_t)P + 1);
    for (int q = 0; q < P; q++) {
        const int d = g.pdim[q], k = g.pk[q];
        std::vector<float> lo(D);
        std::vector<int> first(D), last(D), sbit(D), rcv(D);
        // the home slots by cells: per sender its cell shape and thresholds,
        // and its candidate cells in tiles of 256
        const bool by_cells = cell_mode && k == 0;
        std::vector<int> cls(by_cells ? 4 * (size_t)D : 0), hcprefix(by_cells ? (size_t)D + 1 : 0);
        std::vector<int> ctprefix(by_cells ? (size_t)D + 1 : 0);
        for (int S = 0; S < D; S++) {
            int c[3];
            g.coords(S, c);
            lo[S] = g.b[d][c[d]];
            sbit[S] = c[d] == 0;
            int cr[3] = {c[0], c[1], c[2]};
            cr[d] = (c[d] - 1 + g.n[d]) % g.n[d];
            rcv[S] = g.index(cr);
            if (by_cells) {
                const int nx = g.ncell[0][c[0]], ny = g.ncell[1][c[1]], nz = g.ncell[2][c[2]];
                const int ncd = g.ncell[d][c[d]];
                const int cf = std::min(cfail0, ncd);
                cls[4 * S] = nx;
                cls[4 * S + 1] = ny;
                cls[4 * S + 2] = std::min(cpass0, ncd - 1);
                cls[4 * S + 3] = cf;
                const int hc = (int)((int64_t)nx * ny * nz / ncd * cf);
                hcprefix[S + 1] = hcprefix[S] + hc;
                ctprefix[S + 1] = ctprefix[S] + (hc + 255) / 256;
            }
            if (k == 0) {
                first[S] = by_cells ? p->nhome[S] : 0;
                last[S] = p->ntotal[S];
            } else {
                first[S] = roff_at[S * P + q - 1];
                last[S] = first[S] + rsize_at[S * P + q - 1];
            }
        }
        // slot tiles, numbered sender by sender in slot order: each sender's
        // candidate range cut at its sources' bounds (home slots, then the
        // region of each earlier pulse), then into tiles of kSelTile slots
        std::vector<STile> tiles;
        std::vector<int> tprefix((size_t)D + 1, 0);
        for (int S = 0; S < D; S++) {
            tprefix[S] = (int)tiles.size();
            auto add = [&](int s0, int s1, const int* gid0, const float* xyz0, int home) {
                const int j_lo = std::max(s0, first[S]), j_hi = std::min(s1, last[S]);
                for (int j0 = j_lo; j0 < j_hi; j0 += kSelTile) {
                    STile t;
                    t.S = S;
                    t.j0 = j0;
                    t.j1 = std::min(j0 + kSelTile, j_hi);
                    t.home = home;
                    t.gid = gid0 + (j0 - s0);
                    t.xyz = xyz0 + 3ll * (j0 - s0);
                    tiles.push_back(t);
                }
            };
            add(0, p->nhome[S], p->d_home_gid + hs[S], d_xhome + 3ll * hs[S], 1);
            for (int qq = 0; qq < q; qq++) {
                const size_t it = (size_t)S * P + qq;
                add(roff_at[it], roff_at[it] + rsize_at[it], rgid[qq] + rstart[it],
                    rxyz[qq] + 3ll * rstart[it], 0);
            }
        }
        tprefix[D] = (int)tiles.size();
        const int T = tprefix[D];
        // the pulse's small tables in one copy
        blobs.emplace_back();
        Blob& in = blobs.back();
        const size_t o_lo = in.add(lo), o_sbit = in.add(sbit), o_tprefix = in.add(tprefix);
        const size_t o_tiles = in.add(tiles);
        const int CT = by_cells ? ctprefix[D] : 0;
        std::vector<int> ctile_s((size_t)std::max(CT, 1), 0);
        for (int S = 0; by_cells && S < D; S++)
            for (int b = ctprefix[S]; b < ctprefix[S + 1]; b++)
                ctile_s[b] = S;
        const size_t o_cls = in.add(cls), o_hcprefix = in.add(hcprefix);
        const size_t o_ctprefix = in.add(ctprefix), o_ctile_s = in.add(ctile_s);
        // counting units, sender-major: S's candidate home cells, then its tiles
        std::vector<int> ubase((size_t)D + 1, 0);
        for (int S = 0; S < D; S++)
            ubase[S + 1] = ubase[S] + (by_cells ? hcprefix[S + 1] - hcprefix[S] : 0) +
                           (tprefix[S + 1] - tprefix[S]);
        const int U = ubase[D];
        std::vector<int> snd(D);  // the sender of each receiver
        for (int S = 0; S < D; S++)
            snd[rcv[S]] = S;
        const size_t o_ubase = in.add(ubase);
        const size_t o_rcv = in.add(rcv), o_snd = in.add(snd);
        char* d_in;
        DDH_HIP(in.send(sc, &d_in, s));
        const float* d_lo = (const float*)(d_in + o_lo);
        const int* d_shiftbit = (const int*)(d_in + o_sbit);
        const int* d_tprefix = (const int*)(d_in + o_tprefix);

        SArgs a{};
        a.d = d;
        a.L_d = g.L[d];
        a.rc = g.rc;
        a.tiles = (const STile*)(d_in + o_tiles);
        a.lo = d_lo;
        a.shiftbit = d_shiftbit;
        a.ubase = (const int*)(d_in + o_ubase);
        CArgs ca{};
        if (by_cells) {
            ca.d = d;
            ca.L_d = g.L[d];
            ca.rc = g.rc;
            ca.ctile_s = (const int*)(d_in + o_ctile_s);
            ca.ctprefix = (const int*)(d_in + o_ctprefix);
            ca.hcprefix = (const int*)(d_in + o_hcprefix);
            ca.cls = (const int4*)(d_in + o_cls);
            ca.cellbase = d_cellbase;
            ca.start = d_start;
            ca.home_start = d_hs;
            ca.xhome = d_xhome;
            ca.home_gid = p->d_home_gid;
            ca.lo = d_lo;
            ca.shiftbit = d_shiftbit;
            ca.nblocks = CT;
            a.hcprefix = ca.hcprefix;
        }
        uint32_t *d_ucnt, *d_tbelow, *d_uscan;
        DDH_HIP(sc.alloc(&d_ucnt, (size_t)U + 1));
        DDH_HIP(sc.alloc(&d_tbelow, (size_t)T + 1));
        DDH_HIP(sc.alloc(&d_uscan, (size_t)U + 1));
        if (CT + T > 0)
            hipLaunchKernelGGL(select_count_kernel, dim3(CT + T), dim3(256), 0, s, a, ca, d_tprefix,
                               d_ucnt, d_tbelow);
        DDH_HIP(hipGetLastError());
        const int rcode = scan_exclusive(sc, d_ucnt, U, d_uscan, s);
        if (rcode)
            return rcode;
        // totals and write offsets on the device; the counts go to the host
        // (one event) while the write runs into the room left by earlier builds
        int* d_off;
        DDH_HIP(sc.alloc(&d_off, 3 * (size_t)D + 1));
        uint32_t* d_total = (uint32_t*)(d_off + 3 * (size_t)D);
        hipLaunchKernelGGL(pulse_totals_kernel, dim3(1), dim3(1024), 0, s, a, d_tprefix, D,
                           d_uscan, d_tbelow, d_cnt_send, d_cnt_split, (const int*)(d_in + o_rcv),
                           (const int*)(d_in + o_snd), d_off, d_off + D, d_off + 2 * (size_t)D,
                           d_total);
        DDH_HIP(hipGetLastError());
        void* hcnt;
        DDH_HIP(sc.pinned(&hcnt, 2 * sizeof(int) * (size_t)D));
        DDH_HIP(hipMemcpyAsync(hcnt, d_cnt_send, 2 * sizeof(int) * D, hipMemcpyDeviceToHost, s));
        if (!p->counts_ready)
            DDH_HIP(hipEventCreateWithFlags(&p->counts_ready, hipEventDisableTiming));
        DDH_HIP(hipEventRecord(p->counts_ready, s));
        if (p->selbuf.size() < (size_t)P)
            p->selbuf.resize((size_t)P, {nullptr, 0});
        a.map_pos = d_off;
        a.out_pos = d_off + 2 * (size_t)D;
        a.total = d_total;
        auto place = [&](int qq) {  // the pulse's outputs in its room
            char* base = (char*)p->selbuf[qq].first;
            const size_t cap = p->selbuf[qq].second;
            mapp[qq] = (int*)base;
            rgid[qq] = (int*)(base + sizeof(int) * cap);
            rxyz[qq] = (float*)(base + 2 * sizeof(int) * cap);
            a.cap = (uint32_t)cap;
            a.map_out = mapp[qq];
            a.out_gid = rgid[qq];
            a.out_xyz = rxyz[qq];
            ca.map_pos = a.map_pos;
            ca.map_out = a.map_out;
            ca.out_pos = a.out_pos;
            ca.out_gid = a.out_gid;
            ca.out_xyz = a.out_xyz;
        };
        place(q);
        if (CT + T > 0 && p->selbuf[q].second > 0)
            hipLaunchKernelGGL(select_write_kernel, dim3(CT + T), dim3(256), 0, s, a, ca, d_tprefix,
                               d_uscan);
        DDH_HIP(hipGetLastError());
        std::vector<int> cs(D), cp(D);
        DDH_HIP(hipEventSynchronize(p->counts_ready));
        std::memcpy(cs.data(), hcnt, sizeof(int) * (size_t)D);
        std::memcpy(cp.data(), (int*)hcnt + D, sizeof(int) * (size_t)D);

        // sizes -> offsets; region q of R lands after R's current slots
        mpos[q].assign(D, 0);
        int64_t mt = 0;
        for (int S = 0; S < D; S++) {
            const int it = S * P + q;
            p->send[it] = cs[S];
            p->split[it] = cp[S];
            p->recv[it] = rcv[S];
            p->shift[it] = sbit[S];
            mpos[q][S] = (int)mt;
            mt += cs[S];
        }
        for (int S = 0; S < D; S++) {
            const int R = rcv[S];
            p->roff[S * P + q] = p->ntotal[R];
            roff_at[R * P + q] = p->ntotal[R];
            rsize_at[R * P + q] = cs[S];
            if ((int64_t)p->ntotal[R] + cs[S] > INT32_MAX)
                return fail(DDH_ECAPACITY, "ddh_build_maps: a domain exceeds 2^31 slots");
            p->ntotal[R] += cs[S];
        }
        rsprefix[q].assign((size_t)D + 1, 0);
        for (int R = 0; R < D; R++) {
            rstart[R * P + q] = rsprefix[q][R];
            rsprefix[q][R + 1] = rsprefix[q][R] + rsize_at[R * P + q];
        }
        total[q] = (int)mt;
        if (mt > INT32_MAX)
            return fail(DDH_ECAPACITY, "ddh_build_maps: a pulse exceeds 2^31 entries");
        // no room (the first build of the plan, or the pulse grew by more
        // than the spare quarter): the write above did nothing; grow the
        // room and write again
        if ((size_t)mt > p->selbuf[q].second) {
            const size_t cap = std::max<size_t>(256, (size_t)mt + (size_t)mt / 4);
            DDH_HIP(hipStreamSynchronize(s));  // the skipped write has ended
            if (p->selbuf[q].first)
                DDH_HIP(hipFree(p->selbuf[q].first));
            p->selbuf[q] = {nullptr, 0};
            void* q_buf = nullptr;
            DDH_HIP(hipMalloc(&q_buf, 5 * sizeof(int) * cap));
            p->selbuf[q] = {q_buf, cap};
            place(q);
            if (CT + T > 0)
                hipLaunchKernelGGL(select_write_kernel, dim3(CT + T), dim3(256), 0, s, a, ca,
                                   d_tprefix, d_uscan);
            DDH_HIP(hipGetLastError());
        }
    }

    // ---- 4: final layout
    ph.next("build: layout");
    p->base.assign(D, 0);
    int64_t acc = 0;
    for (int Dm = 0; Dm < D; Dm++) {
        p->base[Dm] = acc;
        acc += p->ntotal[Dm];
    }
    if (acc > INT32_MAX / 3)
        return fail(DDH_ECAPACITY, "ddh_build_maps: layout exceeds the int32 slot range");
    p->n_slots = acc;
    p->n_atoms = n_atoms;
    int64_t nh = 0;
    for (int q = 0; q < P; q++)
        nh += total[q];
    p->n_halo = nh;

    // maps, pulse-major, and a 16-bit copy when every sender-local slot
    // index fits (halves the bytes of the map reads in every pass)
    DDH_HIP(owned_alloc(p, &p->d_maps, (size_t)nh));
    p->map_off.assign(DP, 0);
    MapParts mp{};
    mp.P = P;
    {
        int64_t pb = 0;
        for (int q = 0; q < P; q++) {
            for (int S = 0; S < D; S++)
                p->map_off[S * P + q] = pb + mpos[q][S];
            mp.src[q] = mapp[q];
            mp.begin[q] = pb;
            pb += total[q];
        }
        mp.begin[P] = pb;
    }
    int32_t max_total = 0;
    for (int Dm = 0; Dm < D; Dm++)
        max_total = std::max(max_total, p->ntotal[Dm]);
    if (nh > 0 && max_total <= 65536)
        DDH_HIP(owned_alloc(p, &p->d_maps16, (size_t)nh));
    if (nh > 0)
        hipLaunchKernelGGL(join_maps_kernel, dim3((unsigned)std::min<int64_t>(blocks(nh), 4096)),
                           dim3(256), 0, s, mp, p->d_maps, p->d_maps16);
    DDH_HIP(hipGetLastError());

    // global id per slot, home slot per home atom; pulse of every received
    // slot (rid, 0xff for home slots) for the wait masks
    DDH_HIP(owned_alloc(p, &p->d_slot_gid, (size_t)p->n_slots));
    DDH_HIP(owned_alloc(p, &p->d_home_slot, (size_t)n_atoms));
    // every slot is a home slot (fill_home_kernel writes 0xff) or in one
    // received region (fill_region_kernel writes its pulse)
    DDH_HIP(owned_alloc(p, &p->d_rid, (size_t)p->n_slots));
    std::vector<int> base32(D);
    const int* d_base;
    Blob lay;
    {
        for (int Dm = 0; Dm < D; Dm++)
            base32[Dm] = (int)p->base[Dm];
        // slot bases, and per pulse the region prefix and the receivers'
        // first region slots, in one copy
        const size_t o_base = lay.add(base32);
        std::vector<size_t> o_rs((size_t)P), o_dst((size_t)P);
        std::vector<int> dst(D);
        for (int q = 0; q < P; q++) {
            for (int R = 0; R < D; R++)
                dst[R] = base32[R] + roff_at[R * P + q];
            o_rs[q] = lay.add(rsprefix[q]);
            o_dst[q] = lay.add(dst);
        }
        char* d_lay;
        DDH_HIP(lay.send(sc, &d_lay, s));
        d_base = (const int*)(d_lay + o_base);
        int max_home = 0;
        for (int Dm = 0; Dm < D; Dm++)
            max_home = std::max(max_home, hs[Dm + 1] - hs[Dm]);
        const int cpd = (max_home + kFillTile - 1) / kFillTile;
        if (cpd > 0)
            hipLaunchKernelGGL(fill_home_kernel,
                               dim3((unsigned)std::min<int64_t>((int64_t)D * cpd, kFillMaxBlocks)),
                               dim3(256), 0, s, p->d_home_gid, d_hs, d_base, D, cpd,
                               p->d_slot_gid, p->d_home_slot, p->d_rid);
        for (int q = 0; q < P; q++) {
            int max_region = 0;  // the largest region of the pulse, in chunks
            for (int R = 0; R < D; R++)
                max_region = std::max(max_region, rsize_at[R * P + q]);
            const int cps = (max_region + kSegTile - 1) / kSegTile;
            if (total[q] > 0 && cps > 0)
                hipLaunchKernelGGL(fill_region_kernel,
                                   dim3((unsigned)std::min<int64_t>((int64_t)D * cps, kSegMaxBlocks)),
                                   dim3(256), 0, s, rgid[q], (const int*)(d_lay + o_rs[q]), D, cps,
                                   (const int*)(d_lay + o_dst[q]), p->d_slot_gid, p->d_rid, q);
        }
        DDH_HIP(hipGetLastError());
    }

    // ---- 5: per-pulse chunk tables, counters
    ph.next("build: chunk tables");
    p->pulse.chunk = p->chunk_req > 0 ? p->chunk_req : pulse_chunk(p, true);
    const int chunk1 = p->chunk_req > 0 ? p->chunk_req : pulse_chunk(p, false);
    // every coordinate chunk is a contiguous slice [hb, he) of one map, made
    // on the device from the maps' data
    {
        std::vector<int> info(5 * DP + (size_t)D + (size_t)P);
        int* in = info.data();
        for (size_t it = 0; it < DP; it++) {
            in[it] = p->send[it];
            in[DP + it] = p->recv[it];
            in[2 * DP + it] = (int)p->roff[it];
            in[3 * DP + it] = (int)p->map_off[it];
            in[4 * DP + it] = p->shift[it];
        }
        for (int Dm = 0; Dm < D; Dm++)
            in[5 * DP + Dm] = (int)p->base[Dm];
        for (int q = 0; q < P; q++)
            in[5 * DP + D + q] = g.pdim[q];
        // the tables' chunk counts and first chunks, with the map data, in
        // one copy
        p->pulse1.chunk = chunk1 != p->pulse.chunk ? chunk1 : 0;
        const std::vector<int> pre = pulse_table_counts(p, p->pulse);
        std::vector<int> pre1;
        if (p->pulse1.chunk)
            pre1 = pulse_table_counts(p, p->pulse1);
        Blob tb;
        const size_t o_info = tb.add(info), o_pre = tb.add(pre), o_nch = tb.add(p->pulse.nchunks);
        const size_t o_pre1 = tb.add(pre1), o_nch1 = tb.add(p->pulse1.nchunks);
        char* d_tb;
        DDH_HIP(tb.send(sc, &d_tb, s));
        const int* d_info = (const int*)(d_tb + o_info);
        MapInfo m{};
        m.send = d_info;
        m.recv = d_info + DP;
        m.roff = d_info + 2 * DP;
        m.map_off = d_info + 3 * DP;
        m.shift = d_info + 4 * DP;
        m.base = d_info + 5 * DP;
        m.pdim = d_info + 5 * DP + D;
        for (int d = 0; d < 3; d++)
            m.L[d] = g.L[d];
        m.D = D;
        m.P = P;
        if (int rc = make_pulse_table(p, m, p->pulse, (const int*)(d_tb + o_pre),
                                      (const int*)(d_tb + o_nch), s))
            return rc;
        if (p->pulse1.chunk)
            if (int rc = make_pulse_table(p, m, p->pulse1, (const int*)(d_tb + o_pre1),
                                          (const int*)(d_tb + o_nch1), s))
                return rc;
    }
    ph.next("build: counters");
    const size_t words = (size_t)kCtrlWords + 4 * DP + 2 * (size_t)DDH_MAX_PULSES;
    DDH_HIP(owned_alloc(p, &p->d_ctrl, words));
    DDH_HIP(hipMemsetAsync(p->d_ctrl, 0, sizeof(uint32_t) * words, s));
    p->d_xcnt = p->d_ctrl + kCtrlWords;
    p->d_fcnt = p->d_xcnt + DP;
    p->d_xneed = p->d_fcnt + DP;
    p->d_fneed = p->d_xneed + DP;
    p->d_pflag = p->d_fneed + DP;

    // ---- 6: the fused launch's table, now if the mode may run that launch,
    // else at the first switch to such a mode (prepare_fused); its settings
    // are those of this build
    p->fused.chunk = p->chunk_req > 0 ? p->chunk_req : fused_chunk(p);
    p->fused.wave = p->wave_chunks != 0;
    p->fused.heads_first = p->heads_first != 0;
    p->fused_refined = p->refined_waits != 0;
    const bool fuse_now = p->may_fuse();
    if (fuse_now) {
        ph.next("build: fused table");
        if (int rc = fused_stage(p, sc, s))
            return rc;
    }
    DDH_HIP(hipStreamSynchronize(s));
    p->built = true;
    p->fused_ready = fuse_now;
    p->build_failed = false;
    return DDH_OK;
}

int prepare_fused(Plan* p)
{
    if (!p->built || p->fused_ready)
        return DDH_OK;
    if (!p->capture_stream)
        DDH_HIP(hipStreamCreateWithFlags(&p->capture_stream, hipStreamNonBlocking));
    Scratch sc(p);
    if (int rc = fused_stage(p, sc, p->capture_stream))
        return rc;
    DDH_HIP(hipStreamSynchronize(p->capture_stream));
    p->fused_ready = true;
    return DDH_OK;
}

}  // namespace ddh
