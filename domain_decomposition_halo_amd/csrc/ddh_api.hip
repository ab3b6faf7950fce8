// ddh_api.hip - the C ABI of the staged halo exchange (declared in ddh.h):
// plan lifecycle, geometry and pulse schedule, argument checks, queries.
//
// Source ("the guide"): NVIDIA technical blog "A Practical Guide to
// GPU-Initiated Communication for Molecular Dynamics at Scale". The pulse
// schedule follows "Accelerating GROMACS using Device-initiated Remote Memory
// Access" (dimensions Z, Y, X; one or more pulses per dimension) and
// "Dependency-aware packing" (pulses numbered globally in that order).
#pragma clang fp contract(off)

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>

#include "ddh_internal.h"

namespace ddh {

static thread_local std::string g_last_error;

int fail(int code, const std::string& msg)
{
    g_last_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char* what)
{
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return DDH_EHIP;
}

// Boundaries, sort cells and the pulse schedule of a decomposition.
static int make_geometry(const ddh_params& prm, Geometry& g)
{
    for (int d = 0; d < 3; d++) {
        if (prm.ndom[d] < 1 || prm.ndom[d] > 4096)
            return fail(DDH_EINVAL, "ddh_plan_create: ndom must be in [1, 4096]");
        if (!(prm.box[d] > 0.0f) || !std::isfinite(prm.box[d]))
            return fail(DDH_EINVAL, "ddh_plan_create: box edges must be positive and finite");
        g.n[d] = prm.ndom[d];
        g.L[d] = prm.box[d];
    }
    if (!(prm.rc > 0.0f) || !std::isfinite(prm.rc))
        return fail(DDH_EINVAL, "ddh_plan_create: rc must be positive and finite");
    if ((int64_t)g.n[0] * g.n[1] * g.n[2] > (1 << 20))
        return fail(DDH_EINVAL, "ddh_plan_create: too many domains");
    g.ndom = g.n[0] * g.n[1] * g.n[2];
    g.rc = prm.rc;
    g.cell = prm.cell > 0.0f && std::isfinite(prm.cell) ? prm.cell : 0.0f;
    g.inv_c = g.cell > 0.0f ? (float)(1.0 / (double)g.cell) : 0.0f;
    for (int d = 0; d < 3; d++) {
        g.b[d].resize(g.n[d] + 1);
        for (int i = 0; i < g.n[d]; i++)
            g.b[d][i] = (float)((double)g.L[d] * (double)i / (double)g.n[d]);
        g.b[d][g.n[d]] = g.L[d];
        g.ncell[d].resize(g.n[d]);
        for (int i = 0; i < g.n[d]; i++) {
            int nc = 1;
            if (g.cell > 0.0f)
                nc = (int)std::ceil(((double)g.b[d][i + 1] - (double)g.b[d][i]) / (double)g.cell);
            g.ncell[d][i] = nc < 1 ? 1 : nc;
        }
    }
    g.P = 0;
    for (int d = 2; d >= 0; d--) {
        if (g.n[d] == 1)
            continue;
        double wmin = 1e300, wmax = 0.0;
        for (int i = 0; i < g.n[d]; i++) {
            const double w = (double)g.b[d][i + 1] - (double)g.b[d][i];
            wmin = w < wmin ? w : wmin;
            wmax = w > wmax ? w : wmax;
        }
        if ((double)g.rc > (double)g.L[d] - wmax)
            return fail(DDH_ERANGE, "ddh_plan_create: rc exceeds L - w; the halo would wrap");
        int np = 1;
        while ((double)np * wmin < (double)g.rc)
            np++;
        if (np > g.n[d] - 1)
            return fail(DDH_ERANGE, "ddh_plan_create: relay longer than the domain ring");
        for (int k = 0; k < np; k++) {
            if (g.P >= DDH_MAX_PULSES)
                return fail(DDH_ERANGE, "ddh_plan_create: more than DDH_MAX_PULSES pulses");
            g.pdim[g.P] = d;
            g.pk[g.P] = k;
            g.P++;
        }
    }
    return DDH_OK;
}

static int check_built(const Plan* p)
{
    if (!p)
        return fail(DDH_EINVAL, "null plan");
    if (!p->built)
        return fail(DDH_ESTATE, "the plan has no maps yet (call ddh_build_maps)");
    return DDH_OK;
}

static int check_buffer(const Plan* p, const void* buf, int64_t cap, const char* what)
{
    if (!buf && p->n_slots > 0)
        return fail(DDH_EINVAL, std::string(what) + ": null buffer");
    if (cap < p->n_slots)
        return fail(DDH_ECAPACITY, std::string(what) + ": buffer holds " + std::to_string(cap) +
                                       " slots, the layout needs " + std::to_string(p->n_slots));
    return DDH_OK;
}

}  // namespace ddh

using namespace ddh;

struct ddh_plan : public ddh::Plan {};

extern "C" {

const char* ddh_last_error(void) { return g_last_error.c_str(); }

int ddh_plan_create(const ddh_params* params, ddh_plan** out)
{
    if (!params || !out)
        return fail(DDH_EINVAL, "ddh_plan_create: null argument");
    *out = nullptr;
    Geometry g;
    int rc = make_geometry(*params, g);
    if (rc)
        return rc;
    ddh_plan* p = new (std::nothrow) ddh_plan();
    if (!p)
        return fail(DDH_EINVAL, "ddh_plan_create: out of host memory");
    p->g = g;
    // The plan is bound to the current device. Without one, the geometry and
    // schedule can still be queried; every device call then fails with
    // DDH_EHIP.
    int ncu = 0;
    if (hipGetDevice(&p->device) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, p->device) ==
            hipSuccess &&
        ncu > 0)
        p->n_cu = ncu;
    else
        p->device = -1;
    *out = p;
    return DDH_OK;
}

void ddh_plan_destroy(ddh_plan* p)
{
    if (!p)
        return;
    free_built(p);
    free_scratch(p);
    if (p->capture_stream)
        (void)hipStreamDestroy(p->capture_stream);
    delete p;
}

int ddh_build_maps(ddh_plan* p, const float* xg, int32_t n_atoms, void* stream)
{
    Range range("ddh_build_maps");
    if (!p)
        return fail(DDH_EINVAL, "ddh_build_maps: null plan");
    return build_maps(p, xg, n_atoms, (hipStream_t)stream);
}

int ddh_query(const ddh_plan* p, ddh_layout* out)
{
    if (!p)
        return fail(DDH_EINVAL, "ddh_query: null plan");
    if (!out)
        return fail(DDH_EINVAL, "ddh_query: null output");
    std::memset(out, 0, sizeof(*out));
    out->n_domains = p->g.ndom;
    out->n_pulses = p->g.P;
    out->n_slots = p->n_slots;
    out->n_halo = p->n_halo;
    out->n_atoms = p->n_atoms;
    for (int q = 0; q < p->g.P; q++) {
        out->pulse_dim[q] = p->g.pdim[q];
        out->pulse_k[q] = p->g.pk[q];
    }
    return DDH_OK;
}

int ddh_domain_info(const ddh_plan* p, int32_t dom, int64_t* base, int32_t* n_home, int32_t* n_total)
{
    int rc = check_built(p);
    if (rc)
        return rc;
    if (dom < 0 || dom >= p->g.ndom)
        return fail(DDH_EINVAL, "ddh_domain_info: domain out of range");
    if (base)
        *base = p->base[dom];
    if (n_home)
        *n_home = p->nhome[dom];
    if (n_total)
        *n_total = p->ntotal[dom];
    return DDH_OK;
}

int ddh_pulse_info(const ddh_plan* p, int32_t dom, int32_t pulse, int32_t* send_size, int32_t* split,
                   int32_t* recv_dom, int32_t* recv_offset, int32_t* shift)
{
    int rc = check_built(p);
    if (rc)
        return rc;
    if (dom < 0 || dom >= p->g.ndom || pulse < 0 || pulse >= p->g.P)
        return fail(DDH_EINVAL, "ddh_pulse_info: domain or pulse out of range");
    const int it = dom * p->g.P + pulse;
    if (send_size)
        *send_size = p->send[it];
    if (split)
        *split = p->split[it];
    if (recv_dom)
        *recv_dom = p->recv[it];
    if (recv_offset)
        *recv_offset = p->roff[it];
    if (shift)
        *shift = p->shift[it];
    return DDH_OK;
}

int ddh_copy_maps(const ddh_plan* p, int32_t* maps_dev, int64_t capacity, void* stream)
{
    int rc = check_built(p);
    if (rc)
        return rc;
    if (capacity < p->n_halo)
        return fail(DDH_ECAPACITY, "ddh_copy_maps: buffer smaller than n_halo");
    if (!maps_dev && p->n_halo > 0)
        return fail(DDH_EINVAL, "ddh_copy_maps: null buffer");
    int64_t pos = 0;
    for (int S = 0; S < p->g.ndom; S++)
        for (int q = 0; q < p->g.P; q++) {
            const int it = S * p->g.P + q;
            if (p->send[it] > 0)
                DDH_HIP(hipMemcpyAsync(maps_dev + pos, p->d_maps + p->map_off[it],
                                       sizeof(int32_t) * p->send[it], hipMemcpyDeviceToDevice,
                                       (hipStream_t)stream));
            pos += p->send[it];
        }
    return DDH_OK;
}

static int check_flags_on(const Plan* p, const char* what)
{
    if (!p->flags)
        return fail(DDH_ESTATE, std::string(what) + ": completion flags are off (DDH_TUNE_FLAGS)");
    return DDH_OK;
}

int ddh_flags(const ddh_plan* p, uint32_t** flags_dev)
{
    int rc = check_built(p);
    if (!rc)
        rc = check_flags_on(p, "ddh_flags");
    if (rc)
        return rc;
    if (!flags_dev)
        return fail(DDH_EINVAL, "ddh_flags: null output");
    *flags_dev = p->d_pflag;
    return DDH_OK;
}

int ddh_copy_flags(const ddh_plan* p, uint32_t* flags_dev, void* stream)
{
    int rc = check_built(p);
    if (!rc)
        rc = check_flags_on(p, "ddh_copy_flags");
    if (rc)
        return rc;
    if (!flags_dev)
        return fail(DDH_EINVAL, "ddh_copy_flags: null buffer");
    DDH_HIP(hipMemcpyAsync(flags_dev, p->d_pflag, sizeof(uint32_t) * 2 * DDH_MAX_PULSES,
                           hipMemcpyDeviceToDevice, (hipStream_t)stream));
    return DDH_OK;
}

int ddh_wait_flag(ddh_plan* p, int32_t pass_kind, int32_t pulse, uint32_t epoch, void* stream)
{
    int rc = check_built(p);
    if (!rc)
        rc = check_flags_on(p, "ddh_wait_flag");
    if (rc)
        return rc;
    if (pass_kind != DDH_PASS_COORDS && pass_kind != DDH_PASS_FORCES)
        return fail(DDH_EINVAL, "ddh_wait_flag: pass_kind must be DDH_PASS_COORDS or "
                                "DDH_PASS_FORCES");
    if (pulse < 0 || pulse >= p->g.P)
        return fail(DDH_EINVAL, "ddh_wait_flag: pulse out of range");
    const int idx = (pass_kind == DDH_PASS_FORCES ? DDH_MAX_PULSES : 0) + pulse;
    return enqueue_wait_flag(p, idx, epoch, (hipStream_t)stream);
}

int ddh_local_ids(const ddh_plan* p, int32_t* ids_dev, int64_t capacity, void* stream)
{
    int rc = check_built(p);
    if (rc)
        return rc;
    rc = check_buffer(p, ids_dev, capacity, "ddh_local_ids");
    if (rc)
        return rc;
    if (p->n_slots > 0)
        DDH_HIP(hipMemcpyAsync(ids_dev, p->d_slot_gid, sizeof(int32_t) * p->n_slots,
                               hipMemcpyDeviceToDevice, (hipStream_t)stream));
    return DDH_OK;
}

int ddh_gather_home(ddh_plan* p, const float* xg, float* x, int64_t cap, void* stream)
{
    Range range("ddh_gather_home");
    int rc = check_built(p);
    if (rc)
        return rc;
    if (!xg && p->n_atoms > 0)
        return fail(DDH_EINVAL, "ddh_gather_home: null positions");
    rc = check_buffer(p, x, cap, "ddh_gather_home");
    if (rc)
        return rc;
    return enqueue_gather_home(p, xg, x, (hipStream_t)stream);
}

int ddh_exchange_coords(ddh_plan* p, float* x, int64_t cap, void* stream)
{
    Range range("ddh_exchange_coords");
    int rc = check_built(p);
    if (rc)
        return rc;
    rc = check_buffer(p, x, cap, "ddh_exchange_coords");
    if (rc)
        return rc;
    return enqueue_exchange(p, kOpCoords, x, nullptr, (hipStream_t)stream);
}

int ddh_exchange_forces(ddh_plan* p, float* f, int64_t cap, void* stream)
{
    Range range("ddh_exchange_forces");
    int rc = check_built(p);
    if (rc)
        return rc;
    rc = check_buffer(p, f, cap, "ddh_exchange_forces");
    if (rc)
        return rc;
    return enqueue_exchange(p, kOpForces, nullptr, f, (hipStream_t)stream);
}

int ddh_exchange_step(ddh_plan* p, float* x, float* f, int64_t cap, void* stream)
{
    Range range("ddh_exchange_step");
    int rc = check_built(p);
    if (rc)
        return rc;
    rc = check_buffer(p, x, cap, "ddh_exchange_step (coordinates)");
    if (rc)
        return rc;
    rc = check_buffer(p, f, cap, "ddh_exchange_step (forces)");
    if (rc)
        return rc;
    // the passes may overlap in time, so the arrays must not overlap in memory
    const uintptr_t xb = (uintptr_t)x, fb = (uintptr_t)f;
    const uintptr_t nb = (uintptr_t)p->n_slots * 3u * sizeof(float);
    if (nb > 0 && xb < fb + nb && fb < xb + nb)
        return fail(DDH_EINVAL, "ddh_exchange_step: coordinate and force arrays overlap");
    return enqueue_exchange(p, kOpStep, x, f, (hipStream_t)stream);
}

int ddh_exchange_staged_static(ddh_plan* p, float* x, float* f, int64_t cap, void* stream)
{
    Range range("ddh_exchange_staged_static");
    int rc = check_built(p);
    if (rc)
        return rc;
    if (!x && !f)
        return fail(DDH_EINVAL, "ddh_exchange_staged_static: no coordinate or force array");
    if (x && (rc = check_buffer(p, x, cap, "ddh_exchange_staged_static (coordinates)")))
        return rc;
    if (f && (rc = check_buffer(p, f, cap, "ddh_exchange_staged_static (forces)")))
        return rc;
    const uintptr_t xb = (uintptr_t)x, fb = (uintptr_t)f;
    const uintptr_t nb = (uintptr_t)p->n_slots * 3u * sizeof(float);
    if (x && f && nb > 0 && xb < fb + nb && fb < xb + nb)
        return fail(DDH_EINVAL, "ddh_exchange_staged_static: coordinate and force arrays overlap");
    const int op = (x ? kOpCoords : 0) | (f ? kOpForces : 0);
    return enqueue_staged_static(p, op, x, f, (hipStream_t)stream);
}

int ddh_set_mode(ddh_plan* p, int32_t mode)
{
    if (!p)
        return fail(DDH_EINVAL, "ddh_set_mode: null plan");
    const int32_t base = mode & ~DDH_MODE_GRAPH;
    if (base != DDH_MODE_FUSED && base != DDH_MODE_PULSE && base != DDH_MODE_AUTO &&
        base != DDH_MODE_STAGED)
        return fail(DDH_EINVAL, "ddh_set_mode: unknown mode");
    if (base == DDH_MODE_STAGED && (mode & DDH_MODE_GRAPH))
        return fail(DDH_EINVAL, "ddh_set_mode: DDH_MODE_STAGED waits on the host and cannot "
                                "be replayed from a graph");
    const int32_t old = p->mode;
    p->mode = mode;
    // a build made under a mode that never runs the fused launch did not
    // make its table: make it now if the new mode may run it
    if (p->built && !p->fused_ready && p->may_fuse()) {
        if (int rc = prepare_fused(p)) {
            p->mode = old;
            return rc;
        }
    }
    return DDH_OK;
}

int ddh_check(ddh_plan* p, void* stream)
{
    Range range("ddh_check");
    if (!p)
        return fail(DDH_EINVAL, "ddh_check: null plan");
    DDH_HIP(hipStreamSynchronize((hipStream_t)stream));
    if (!p->d_ctrl)
        return DDH_OK;
    uint32_t word = 0;
    DDH_HIP(hipMemcpy(&word, p->d_ctrl + kCtrlError, sizeof(word), hipMemcpyDeviceToHost));
    if (word) {
        DDH_HIP(hipMemset(p->d_ctrl + kCtrlError, 0, sizeof(word)));
        return fail((int)word, "a device-side wait exceeded its spin limit");
    }
    return DDH_OK;
}

int ddh_tune(ddh_plan* p, int32_t key, int64_t value)
{
    if (!p)
        return fail(DDH_EINVAL, "ddh_tune: null plan");
    // captured graphs hold the launch arguments of the old settings
    for (auto& kv : p->graphs)
        (void)hipGraphExecDestroy(kv.second);
    p->graphs.clear();
    switch (key) {
    case DDH_TUNE_CHUNK:
        if (value != 0 && (value < 64 || value > 65536))
            return fail(DDH_EINVAL, "ddh_tune: chunk must be 0 or in [64, 65536]");
        p->chunk_req = (int)((value + 63) / 64 * 64);
        return DDH_OK;
    case DDH_TUNE_GRID:
        if (value < 0 || value > (1 << 20))
            return fail(DDH_EINVAL, "ddh_tune: grid out of range");
        p->grid_req = (int)value;
        return DDH_OK;
    case DDH_TUNE_SPIN_LIMIT:
        if (value < 1 || value > 0xffffffffll)
            return fail(DDH_EINVAL, "ddh_tune: spin limit out of range");
        p->spin_limit = (uint32_t)value;
        return DDH_OK;
    case DDH_TUNE_FORCE_TIMEOUT:
        p->force_timeout = value != 0;
        return DDH_OK;
    case DDH_TUNE_REFINED_WAITS:
        p->refined_waits = value != 0;
        return DDH_OK;
    case DDH_TUNE_BLOCK:
        if (value != 0 && value != 256 && value != 512 && value != 1024)
            return fail(DDH_EINVAL, "ddh_tune: block must be 0, 256, 512 or 1024");
        p->block_req = (int)value;
        return DDH_OK;
    case DDH_TUNE_TRACE:
        p->trace = (uint64_t*)(uintptr_t)value;
        return DDH_OK;
    case DDH_TUNE_FLAGS:
        if (value != 0 && value != 1)
            return fail(DDH_EINVAL, "ddh_tune: flags must be 0 or 1");
        p->flags = (int)value;
        return DDH_OK;
    case DDH_TUNE_STATIC_FIRST:
        if (value != 0 && value != 1)
            return fail(DDH_EINVAL, "ddh_tune: static-first must be 0 or 1");
        p->static_first = (int)value;
        return DDH_OK;
    case DDH_TUNE_NARROW_MAPS:
        if (value != 0 && value != 1)
            return fail(DDH_EINVAL, "ddh_tune: narrow-maps must be 0 or 1");
        p->narrow_maps = (int)value;
        return DDH_OK;
    case DDH_TUNE_WAVE_CHUNKS:
        if (value != 0 && value != 1)
            return fail(DDH_EINVAL, "ddh_tune: wave-chunks must be 0 or 1");
        p->wave_chunks = (int)value;
        return DDH_OK;
    case DDH_TUNE_EXIT_PUBLISH:
        if (value < 0 || value > 2)
            return fail(DDH_EINVAL, "ddh_tune: exit-publish must be 0, 1 or 2");
        p->exit_publish = (int)value;
        return DDH_OK;
    case DDH_TUNE_HEADS_FIRST:
        if (value != 0 && value != 1)
            return fail(DDH_EINVAL, "ddh_tune: heads-first must be 0 or 1");
        p->heads_first = (int)value;
        return DDH_OK;
    case DDH_TUNE_LDS_STAGE:
        if (value < 0 || value > 2)
            return fail(DDH_EINVAL, "ddh_tune: lds-stage must be 0, 1 or 2");
        p->lds_stage = (int)value;
        return DDH_OK;
    case DDH_TUNE_PAD_MAPS:
        if (value < 0 || value > 2)
            return fail(DDH_EINVAL, "ddh_tune: pad-maps must be 0, 1 or 2");
        p->pad_maps = (int)value;
        return DDH_OK;
    case DDH_TUNE_HOME_SORT:
        if (value < 0 || value > 2)
            return fail(DDH_EINVAL, "ddh_tune: home-sort must be 0, 1 or 2");
        p->home_sort = (int)value;
        return DDH_OK;
    default:
        return fail(DDH_EINVAL, "ddh_tune: unknown key");
    }
}

}  // extern "C"
