/*
 * ddh.h - staged halo exchange of a domain-decomposed MD step on one MI355X.
 *
 * Every domain of a spatial decomposition is a virtual rank whose atoms live
 * in one flat device array of float3 records. The library builds the per-pulse
 * index maps and then runs, as hand-written gfx950 kernels,
 *   - the coordinate pass: pulse by pulse Z -> Y -> X, each pulse gathering
 *     boundary records through its index map (with the periodic shift) and
 *     writing them straight into the receiving domain's slots, later pulses
 *     relaying records received in earlier ones;
 *   - the force pass: the same pulses in reverse order X -> Y -> Z, each
 *     scatter-adding the receiver's halo forces back through the map.
 *
 * Source ("the guide"): NVIDIA technical blog "A Practical Guide to
 * GPU-Initiated Communication for Molecular Dynamics at Scale". The sections
 * that define each call are named in its comment.
 *
 * Conventions for every call:
 *   - Return value: DDH_OK (0) or a negative DDH_E* code; no exception or
 *     abort ever crosses this boundary. ddh_last_error() gives a text for the
 *     last failure on the calling thread.
 *   - Pointers marked _dev are device pointers on the plan's device; _host
 *     pointers are host memory. The caller owns every buffer it passes and
 *     keeps it alive until the enqueued work has finished.
 *   - stream is a hipStream_t (NULL = the default stream), passed as void*.
 *     Exchange calls only enqueue work and return at once; they never wait
 *     for the device. Map building waits (it must learn the sizes).
 *   - Arrays of coordinates and forces are float32 AoS: slot s occupies
 *     floats [3s, 3s+3). "capacity_slots" is the number of slots the caller's
 *     buffer holds; a call rejects a buffer smaller than the plan's layout
 *     with DDH_ECAPACITY before enqueuing anything.
 *   - A plan is not thread-safe: use one plan per host thread and stream.
 *
 * Layout of the flat slot array (the guide, "From MPI baseline to optimized
 * GPU-native halo exchange": received coordinates land at the receiver's
 * offset and are used in place). Domain D = ix + nx * (iy + ny * iz) owns
 * slots [base_D, base_D + n_total_D): first its n_home_D home atoms, ordered
 * by sort cell, then by class, then by global id (the class, at
 * ddh_build_maps, keeps together the atoms of a cell that each dimension's
 * first pulse sends), then one contiguous received region per pulse in global
 * pulse order.
 */
#ifndef DDH_H
#define DDH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ error codes */
#define DDH_OK 0
#define DDH_EINVAL (-1)    /* bad argument: null pointer, ndom < 1, rc <= 0,
                              box <= 0, a position outside [0, L) or NaN */
#define DDH_ERANGE (-2)    /* rc > L_d - max width on a decomposed dimension
                              (the halo would wrap onto itself), or more
                              pulses than DDH_MAX_PULSES */
#define DDH_ECAPACITY (-3) /* caller buffer smaller than the layout needs, or
                              a layout beyond 2^31 - 1 slots */
#define DDH_EHIP (-4)      /* a HIP runtime call failed; see ddh_last_error */
#define DDH_ETIMEOUT (-5)  /* a device-side wait exceeded its spin limit */
#define DDH_ENOTIMPL (-6)  /* not implemented */
#define DDH_ESTATE (-7)    /* call out of order (e.g. exchange before build) */

#define DDH_MAX_PULSES 16

/* ---------------------------------------------------------------- types */
typedef struct ddh_params {
    int32_t ndom[3]; /* virtual domains along x, y, z (each >= 1) */
    float box[3];    /* periodic box edges L_x, L_y, L_z (nm) */
    float rc;        /* halo cutoff (nm), > 0 */
    float cell;      /* edge of the cells home atoms are sorted by (nm);
                        <= 0: one cell per domain */
    int32_t flags;   /* reserved, pass 0 */
} ddh_params;

typedef struct ddh_layout {
    int32_t n_domains;
    int32_t n_pulses;                  /* total pulses, global order */
    int64_t n_slots;                   /* slots of the flat array */
    int64_t n_halo;                    /* sum of every map's size per pass */
    int32_t n_atoms;                   /* atoms given to ddh_build_maps */
    int32_t pulse_dim[DDH_MAX_PULSES]; /* dimension of pulse p: 0=x 1=y 2=z */
    int32_t pulse_k[DDH_MAX_PULSES];   /* index of pulse p in its dimension */
} ddh_layout;

typedef struct ddh_plan ddh_plan;

/* Execution modes for the exchange calls (ddh_set_mode). */
#define DDH_MODE_FUSED 0   /* one launch per call: all pulses chained on
                              per-map device counters */
#define DDH_MODE_PULSE 1   /* one launch per pulse, ordered by the stream,
                              then one launch that publishes per-pulse flags */
#define DDH_MODE_AUTO 2    /* default: PULSE, except for a call that is
                              enqueued eagerly (the stream is not capturing
                              and DDH_MODE_GRAPH is off) on a pass of at most
                              DDH_AUTO_FUSED_MAX halo atoms, which runs FUSED:
                              there the host's cost per launch dominates */
#define DDH_MODE_STAGED 3  /* host-orchestrated baseline ("From MPI baseline
                              to optimized GPU-native halo exchange"): per
                              pulse a pack launch into a staging buffer, a
                              host wait, one device-to-device copy per sender,
                              a host wait (forces: the reverse, with an unpack
                              launch that adds). The call returns when the
                              pass is complete; it cannot be captured
                              (DDH_EINVAL with DDH_MODE_GRAPH or on a
                              capturing stream). Same results as the others. */
#define DDH_MODE_GRAPH 16  /* OR-able: replay the call's launches from a
                              captured hipGraph */
#define DDH_AUTO_FUSED_MAX 200000

/* ------------------------------------------------------------- lifecycle */

/*
 * Create a plan for one decomposition. Validates the parameters, computes the
 * domain boundaries b_d[i] = fl32(L_d * i / n_d) and the pulse schedule:
 * dimensions Z, then Y, then X ("Accelerating GROMACS using Device-initiated
 * Remote Memory Access"), ceil-style pulse count per dimension (the smallest
 * k with k * min width >= rc), none for a dimension with one domain.
 * Uses the current HIP device. Errors: DDH_EINVAL, DDH_ERANGE, DDH_EHIP.
 */
int ddh_plan_create(const ddh_params *params, ddh_plan **out);

/* Release every device and host resource of the plan (NULL is a no-op).
   Library utility: the guide defines no such call. */
void ddh_plan_destroy(ddh_plan *plan);

/* Text for the last failure on the calling thread ("" if none). Library
   utility: the guide defines no such call. */
const char *ddh_last_error(void);

/* ------------------------------------------------------------- map build */

/*
 * Build the halo maps from global positions x_global_dev[n_atoms][3]
 * (device, float32, every coordinate in [0, L)). Runs on `stream` and waits
 * for it. Steps: assign each atom to the domain whose half-open interval
 * holds it in every dimension; order each domain's home atoms by sort cell,
 * class and global id. Cells go row by row (row = cy + ncy * cz), along x
 * upward in even rows and downward in odd ones. An atom's class comes from
 * the slab tests of the first pulses, bit d = [fl(x_d - lo_d) < rc] (m): 7 -
 * m in cells whose x index differs from px = floor(fl(rc * fl(1 / cell))) by
 * an even number in an even row or an odd number in an odd row, else m. The
 * guide fixes neither order; these keep each pulse's atoms of a cell that
 * its slab cuts in one run, adjacent to the next cell's run along the walk,
 * and join the x pulse's cells of neighbouring rows, so the pulses' gathers
 * touch fewer memory lines. Then for every pulse p (dimension d) and sender
 * S choose the candidate slots (k == 0: home plus all slots received in
 * earlier pulses; k >= 1: the slots received in the previous pulse of d),
 * keep those with fl(x_d - lo_d(S)) < rc in increasing slot order, and
 * deliver them to the -d neighbour. Cell-sorted home atoms, slab selection and multi-pulse relay
 * follow "Accelerating GROMACS using Device-initiated Remote Memory Access"
 * and "Enabling parallelism across pulses through kernel fusion" (the
 * dependency offset of each map is the sender's home count).
 * Replaces any previous maps of the plan. Meant to run at every
 * neighbour-search step: the plan keeps its device memory and reuses it in
 * later builds while it is large enough (ddh_plan_destroy releases it).
 * The library's own graphs (DDH_MODE_GRAPH) are recaptured after a build,
 * but exchange calls captured into a caller's graph keep the launch shapes
 * and the tables of the build they were captured after: recapture them
 * after every ddh_build_maps.
 * Errors: DDH_EINVAL (bad pointer or position, more than 2^29 atoms),
 * DDH_ECAPACITY (layout too large), DDH_EHIP.
 */
int ddh_build_maps(ddh_plan *plan, const float *x_global_dev, int32_t n_atoms, void *stream);

/* Layout summary: the pulse schedule (dimensions Z, then Y, then X, with
   several pulses in a dimension narrower than the cutoff: "Accelerating
   GROMACS using Device-initiated Remote Memory Access") and the slot counts
   of the flat array in which received records land at the receiver's atom
   offset ("From MPI baseline to optimized GPU-native halo exchange"). Before
   ddh_build_maps only the domain count and the pulse schedule are set (slot,
   halo and atom counts are 0). Host output. Errors: DDH_EINVAL. */
int ddh_query(const ddh_plan *plan, ddh_layout *out);

/* Slot range of domain dom: base, home count, total count (host outputs).
   The range is the domain's own coordinate array of "From MPI baseline to
   optimized GPU-native halo exchange": its home atoms first, then the
   records received in each pulse at their atom offsets. Errors: DDH_EINVAL
   (bad domain), DDH_ESTATE (no build yet). */
int ddh_domain_info(const ddh_plan *plan, int32_t dom, int64_t *base, int32_t *n_home,
                    int32_t *n_total);

/*
 * Map metadata of sender dom in pulse p (host outputs, any may be NULL):
 * send_size (entries), split (entries below the sender's home count: the
 * independent head), recv_dom (receiving domain), recv_offset (first slot of
 * the region inside the receiver, relative to its base), shift (1 if the
 * pulse's component gets + L at this sender). These are the per-pulse
 * arguments of the guide's pack-and-send kernels (send size, receiving rank,
 * atom offset in the receiver: "From MPI baseline to optimized GPU-native
 * halo exchange", "Replacing host-side communication with NVSHMEM") and the
 * dependency offset of "Enabling parallelism across pulses through kernel
 * fusion". Errors: DDH_EINVAL (bad domain or pulse), DDH_ESTATE.
 */
int ddh_pulse_info(const ddh_plan *plan, int32_t dom, int32_t pulse, int32_t *send_size,
                   int32_t *split, int32_t *recv_dom, int32_t *recv_offset, int32_t *shift);

/*
 * Copy every map (sender-local slot indices, int32) to maps_dev, concatenated
 * with the sender outer and the pulse inner; capacity is in int32 elements
 * and must be >= n_halo. These are the index maps through which the pack
 * kernel of "From MPI baseline to optimized GPU-native halo exchange"
 * gathers its boundary atoms (entries in increasing slot order). The caller
 * owns maps_dev. Asynchronous on stream. Errors: DDH_EINVAL, DDH_ECAPACITY,
 * DDH_ESTATE, DDH_EHIP.
 */
int ddh_copy_maps(const ddh_plan *plan, int32_t *maps_dev, int64_t capacity, void *stream);

/*
 * Per-pulse completion flags ("From MPI baseline to optimized GPU-native halo
 * exchange": a signal counter per pulse; "Dependency-aware packing": the
 * last arrival stores the flag). *flags_dev receives the device address of
 * the plan's uint32[2 * DDH_MAX_PULSES]: word p counts the coordinate passes
 * whose pulse p has been delivered to every receiver, word DDH_MAX_PULSES + p
 * the force passes whose pulse-p adds are all done, since the last
 * ddh_build_maps (which zeroes them). The words only grow (modulo 2^32). A
 * kernel on another stream may poll word p (agent-scope atomic load) until it
 * reaches the pass it needs, then acquire (agent-scope fence) and read the
 * pulse's region. When each word is published:
 *   - DDH_MODE_PULSE: pulse q's words when the call's next launch starts
 *     (in a step, pulse q of the coordinates and P-1-q of the forces share a
 *     launch), the last launch's words by the call's final one-wave launch;
 *   - DDH_MODE_FUSED: every pulse's words when the launch's last work-group
 *     leaves;
 *   - DDH_MODE_STAGED: every pulse's words at the end of the call.
 * The array belongs to the plan and lives until ddh_plan_destroy or the next
 * ddh_build_maps.
 */
int ddh_flags(const ddh_plan *plan, uint32_t **flags_dev);

/* Copy the 2 * DDH_MAX_PULSES flag words into flags_dev (device, uint32),
   ordered on stream after the work enqueued before it. Asynchronous. */
int ddh_copy_flags(const ddh_plan *plan, uint32_t *flags_dev, void *stream);

#define DDH_PASS_COORDS 0
#define DDH_PASS_FORCES 1

/*
 * Make the work enqueued on stream after this call wait until pulse `pulse`
 * of the coordinate (DDH_PASS_COORDS) or force (DDH_PASS_FORCES) pass has
 * completed `epoch` times (its flag word reaches epoch, modulo 2^32), and
 * see the records it delivered: a one-wave wait on the device, ending with
 * an agent-scope acquire ("From MPI baseline to optimized GPU-native halo
 * exchange": the receiver's wait on the pulse's signal). It lets work that
 * needs only pulse p's halo, on another stream, start before the rest of the
 * exchange. The wait is bounded by DDH_TUNE_SPIN_LIMIT polls; on expiry
 * ddh_check reports DDH_ETIMEOUT and the stream goes on. Asynchronous;
 * DDH_EINVAL for a bad pass kind or pulse.
 */
int ddh_wait_flag(ddh_plan *plan, int32_t pass_kind, int32_t pulse, uint32_t epoch, void *stream);

/* Global atom id of every slot (int32[n_slots], device; capacity in int32
   elements). Library utility for callers that map slots back to atoms; the
   guide defines no such call. Asynchronous. Errors: DDH_EINVAL,
   DDH_ECAPACITY, DDH_ESTATE. */
int ddh_local_ids(const ddh_plan *plan, int32_t *ids_dev, int64_t capacity, void *stream);

/*
 * Fill the home slots of x_local_dev from x_global_dev (the array given to
 * ddh_build_maps or any array of the same atoms). Halo slots are untouched.
 * Library utility: the guide takes each rank's home coordinates as given;
 * this call places a caller's positions into the layout. Asynchronous.
 * Errors: DDH_EINVAL, DDH_ECAPACITY, DDH_ESTATE.
 */
int ddh_gather_home(ddh_plan *plan, const float *x_global_dev, float *x_local_dev,
                    int64_t capacity_slots, void *stream);

/* ----------------------------------------------------------- exchanges */

/*
 * Coordinate pass ("From MPI baseline to optimized GPU-native halo exchange",
 * "Optimizing for efficient transfers across NVIDIA NVLink-connected GPUs",
 * "Dependency-aware packing"): for pulses in increasing order, every sender S
 * copies x[base_S + map[i]] to x[base_R + recv_offset + i], adding L_d to
 * component d when S sits at index 0 of d. Reads home slots, writes every
 * halo slot; the result is bit-identical to the sequential pulse order.
 * Asynchronous on stream.
 */
int ddh_exchange_coords(ddh_plan *plan, float *x_local_dev, int64_t capacity_slots,
                        void *stream);

/*
 * Force pass ("From MPI baseline to optimized GPU-native halo exchange",
 * "Force halo exchange: Reversing the dependency chain"): for pulses in
 * decreasing order, every sender S adds f[base_R + recv_offset + i] into
 * f[base_S + map[i]] (fp32, in place). Each slot receives its adds in
 * decreasing pulse order, so the result is bit-identical to the sequential
 * reverse pass over the whole array, halo slots included. Asynchronous.
 */
int ddh_exchange_forces(ddh_plan *plan, float *f_local_dev, int64_t capacity_slots,
                        void *stream);

/*
 * One coordinate pass and one force pass in a single launch (fused mode) or
 * one launch sequence (pulse mode: coordinate pulse q and force pulse P-1-q
 * share a launch). The passes touch different arrays and may overlap in
 * time; the results are those of ddh_exchange_coords then
 * ddh_exchange_forces. The two arrays must not overlap (DDH_EINVAL).
 * Asynchronous.
 */
int ddh_exchange_step(ddh_plan *plan, float *x_local_dev, float *f_local_dev,
                      int64_t capacity_slots, void *stream);

/*
 * The host-orchestrated exchange of DDH_MODE_STAGED (the same launches,
 * copies and host waits, and the same results, whatever mode the plan is
 * set to), for callers that cannot allocate device memory: harnesses that
 * forbid it and tight serving loops. The staging buffer that DDH_MODE_STAGED
 * allocates at its first call is here a static device array of the library
 * (DDH_STATIC_STAGE_BYTES, one per device, held until the process ends), so
 * the call allocates nothing. x_local_dev (coordinate pass) and/or
 * f_local_dev (force pass, after the coordinate pass when both are given)
 * may be NULL, not both; the two must not overlap. The plan's device must be
 * current. Returns when the passes are complete; it cannot be captured.
 * Every call on a device shares that device's array: calls that overlap in
 * time on one device (other host threads, other plans) race. Errors:
 * DDH_EINVAL, DDH_ESTATE, DDH_ECAPACITY (a buffer smaller than the layout,
 * or 12 * n_halo above DDH_STATIC_STAGE_BYTES), DDH_EHIP.
 */
#define DDH_STATIC_STAGE_BYTES 67108864 /* 64 MiB */
int ddh_exchange_staged_static(ddh_plan *plan, float *x_local_dev, float *f_local_dev,
                               int64_t capacity_slots, void *stream);

/* Select DDH_MODE_FUSED, DDH_MODE_PULSE or DDH_MODE_AUTO, optionally
   | DDH_MODE_GRAPH, or DDH_MODE_STAGED alone: the execution forms of
   "Enabling parallelism across pulses through kernel fusion" (one launch),
   "Replacing host-side communication with NVSHMEM" (one launch per pulse)
   and "From MPI baseline to optimized GPU-native halo exchange" (host
   orchestrated). All give the same results. A build makes the single
   launch's chunk table only when the plan's mode may run that launch
   (FUSED, or AUTO without GRAPH on at most DDH_AUTO_FUSED_MAX halo atoms);
   switching a built plan to such a mode makes it then, with the settings of
   that build, on a stream of the plan's own, and waits for it. Errors:
   DDH_EINVAL, DDH_EHIP (the mode is then left unchanged). */
int ddh_set_mode(ddh_plan *plan, int32_t mode);

/*
 * Wait for stream, then read and clear the plan's device error word.
 * Returns DDH_OK, DDH_ETIMEOUT (a device wait hit its spin limit: the
 * results of that call are not valid) or DDH_EHIP. Library utility: the
 * guide's waits on signals ("Dependency-aware packing") are unbounded; the
 * library bounds them and reports an expiry here.
 */
int ddh_check(ddh_plan *plan, void *stream);

/* -------------------------------------------------------------- tuning */
#define DDH_TUNE_CHUNK 1        /* map entries per work chunk (64..65536, rounded
                                   to a multiple of 64); 0 = automatic */
#define DDH_TUNE_GRID 2         /* workgroups of a fused launch; 0 = automatic
                                   (one per compute unit, at most one per
                                   chunk) */
#define DDH_TUNE_SPIN_LIMIT 3   /* polls before a device wait gives up */
#define DDH_TUNE_FORCE_TIMEOUT 4 /* 1: every dependent wait of the fused mode
                                    targets a value no one writes, so it ends
                                    at the spin limit (tests of the timeout
                                    path); pulse mode has no device waits */
#define DDH_TUNE_REFINED_WAITS 5 /* 1 (default): a chunk waits only on the
                                    pulses its entries reference; 0: on all
                                    earlier (coordinates) / later (forces) */

#define DDH_TUNE_TRACE 6          /* value: device address of a uint64 buffer of
                                    2 * 64 * (work-groups of a fused launch)
                                    words, or 0 (off). Thread 0 of every
                                    work-group of a fused launch logs its events
                                    (claim, head done, wait done, chunk done,
                                    flag published, exit) as pairs
                                    (code << 32 | info, 100 MHz wall-clock
                                    ticks), up to 64 per work-group. The caller
                                    owns the buffer and sizes it for the grid
                                    (DDH_TUNE_GRID); the buffer is not cleared. */

#define DDH_TUNE_BLOCK 7           /* work-group width of the exchange launches:
                                    0 (automatic: fused 1024; per-pulse
                                    256), 256, 512 (per-pulse launches; the
                                    fused launch then takes 256) or 1024 */

#define DDH_TUNE_STATIC_FIRST 8    /* fused mode: 0 (default) every work-group
                                    claims its tickets in start order, so no
                                    chunk waits on one that has not started,
                                    whatever else runs on the GPU; 1 work-group
                                    b of a grid of at most one per compute
                                    unit starts with ticket b unclaimed (saves
                                    one atomic per work-group, but only safe
                                    while the launch has the GPU to itself) */

#define DDH_TUNE_FLAGS 9           /* 1 (default): every call publishes the
                                    per-pulse completion flags (ddh_flags);
                                    0: calls skip it (per-pulse mode: no final
                                    one-wave launch; fused mode: no exit
                                    publication) and ddh_flags, ddh_copy_flags
                                    and ddh_wait_flag return DDH_ESTATE. The
                                    flag words count the passes run with flags
                                    on. */

#define DDH_TUNE_NARROW_MAPS 10    /* 1 (default): when every domain has at
                                    most 65536 slots, the exchange kernels read
                                    a 16-bit copy of the maps (2 bytes per
                                    entry instead of 4; same entries, same
                                    results); 0: they read the 32-bit maps */

#define DDH_TUNE_WAVE_CHUNKS 11    /* fused mode: 0 (default) work-groups
                                    claim chunks and take barriers around
                                    their waits; 1 every wavefront is an
                                    independent worker: chunks are contiguous
                                    map slices (default 1024 entries), a
                                    wavefront waits only when its slice holds
                                    dependent entries and releases its own
                                    records, with no work-group barrier (the
                                    guide's per-warp pipelining). Takes effect
                                    at the next build. */

#define DDH_TUNE_HOME_SORT 12      /* how the build orders the home atoms (by
                                    domain, cell, class, then global id; the
                                    result is the same): 0 (default) automatic, the
                                    partition sort where its tables fit (at
                                    most 2048 domains and 4096 sort cells per
                                    domain), else the counting sort; 1 the
                                    counting sort (per-atom device atomics,
                                    then a per-cell sort); 2 the partition
                                    sort (per-block domain histograms and one
                                    block per domain counting by cell, all in
                                    LDS; the build fails with DDH_EINVAL where
                                    it does not fit). Takes effect at the
                                    next build. */

#define DDH_TUNE_EXIT_PUBLISH 13   /* per-pulse mode with completion flags:
                                    0 (default) automatic; 1 the call's last
                                    launch publishes its pulses' flags when
                                    its last block leaves (every block
                                    releases its records first); 2 a one-wave
                                    launch after the last pulse launch
                                    publishes them */

#define DDH_TUNE_PAD_MAPS 14       /* per-pulse mode: 0 (default) automatic;
                                    1 every block loads its first map entries
                                    from a chunk-aligned copy of the maps
                                    before its chunk descriptor arrives (reads
                                    the copy's zero padding too); 2 it loads
                                    the descriptor first, then only the
                                    chunk's own entries. The copy of the
                                    32-bit maps exists only when the build
                                    ran with DDH_TUNE_NARROW_MAPS 0 (or the
                                    maps have no 16-bit copy); otherwise a
                                    later switch to 32-bit maps reads them as
                                    in 2. */

#define DDH_TUNE_HEADS_FIRST 15    /* fused mode: 0 (default) a coordinate
                                    chunk packs a slice of its map's
                                    independent head, waits, then packs a
                                    slice of its dependent tail; 1 heads and
                                    tails are chunks of their own, and every
                                    head (pulse order) is ticketed before any
                                    tail (pulse order), so no head waits.
                                    Same results. Takes effect at the next
                                    build. */

#define DDH_TUNE_LDS_STAGE 16      /* per-pulse and fused modes: 0 (default) coordinate
                                    records are stored from registers (one
                                    12-byte store per lane); 1 each
                                    wavefront stages its 64 gathered records
                                    in LDS and stores the contiguous run in
                                    16-byte aligned groups (the guide's
                                    shared-memory staging before its bulk
                                    stores, "NVLink path: TMA-based direct
                                    stores"); 2 the same, with the records
                                    gathered straight into LDS by the LDS's
                                    own loads (global_load_lds). Applies to
                                    the per-pulse launches' 256-wide blocks
                                    and the fused launch (1024-wide
                                    work-groups and wavefront workers); same
                                    results. */

/* Set a tuning knob; takes effect at the next build (CHUNK, WAVE_CHUNKS,
   HOME_SORT, HEADS_FIRST, REFINED_WAITS: the single launch's table keeps the
   values of the build it belongs to, also when ddh_set_mode makes it later)
   or call. Library utility: the guide defines no such call.
   Errors: DDH_EINVAL (unknown key or value out of range). */
int ddh_tune(ddh_plan *plan, int32_t key, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* DDH_H */
