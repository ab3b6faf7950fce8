/*
 * ddh_oracle.c - CPU oracle for the staged (pulse-by-pulse) halo exchange of a
 * domain-decomposed molecular-dynamics step.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously correct
 * reference that the HIP library is checked against. Only the test suite, the
 * smoke check and the bench's CPU-baseline leg may load it. The HIP library
 * never links, includes or calls it, and it shares no code with the library.
 *
 * Source ("the guide"): NVIDIA technical blog "A Practical Guide to
 * GPU-Initiated Communication for Molecular Dynamics at Scale". Sections are
 * cited by their titles.
 *
 * What the guide fixes, and where:
 *  - "Accelerating GROMACS using Device-initiated Remote Memory Access":
 *    boundary atoms are relayed through intermediate domains within each
 *    dimension over one or more pulses; the phases run Z, then Y, then X;
 *    each pulse gathers its boundary atoms into one contiguous region.
 *  - "From MPI baseline to optimized GPU-native halo exchange": the pack is
 *    an index-map gather of float3 records; received coordinates land in the
 *    receiver's coordinate array at a per-pulse offset and are used in place;
 *    forces travel the same way backwards (X, then Y, then Z) and are
 *    scatter-added through the same index map into the full force array.
 *  - "Enabling parallelism across pulses through kernel fusion": entries of
 *    a pulse's map below the dependency offset (home atoms) need nothing from
 *    earlier pulses; entries at or above it are atoms forwarded from earlier
 *    pulses.
 *
 * Readings taken where the guide is silent:
 *  - one-sided halo: in every pulse a domain sends to its -d neighbour and
 *    receives from its +d neighbour, so each domain's halo lies on its +d side;
 *  - candidates of pulse k of dimension d: for k == 0 the sender's home slots
 *    and every slot it received in earlier pulses, for k >= 1 only the slots
 *    it received in pulse k-1 of the same dimension;
 *  - selection: slot j is sent iff fl(x_j[d] - lo_d(S)) < rc (fp32 subtract,
 *    strict compare), so the halo is box-shaped with no corner rounding;
 *  - periodic shift at the sender: component d gets + L_d (fp32 add) iff the
 *    sender sits at index 0 of dimension d;
 *  - the dependency offset of a map is the sender's home-atom count;
 *  - pulses per dimension: the smallest k >= 1 with k * min_i w_d[i] >= rc,
 *    and a configuration with rc > L_d - max_i w_d[i], or needing more than
 *    n_d - 1 pulses, is rejected (the halo would wrap onto itself);
 *  - boundaries b_d[i] = fl32(L_d * i / n_d) evaluated in double, intervals
 *    half-open [b_d[i], b_d[i+1]);
 *  - home atoms are ordered by sort cell, then by class, then by global id;
 *    the cell index in a dimension is floor(fl(fl(x - lo) * fl32(1/c)))
 *    clamped to [0, ceil((hi - lo) / c) - 1] (c <= 0: one cell per domain,
 *    index 0); cells go row by row, row = cy + ncy * cz, and along x within
 *    a row, upward in even rows and downward in odd ones (a serpentine), key
 *    = x' + ncx * row with x' = cx or ncx - 1 - cx. The rows' cells below
 *    the x cut then meet those of the next row;
 *  - the class orders a cell's atoms by the first pulses that send them:
 *    m = sum over d of 2^d [fl(x_d - lo_d) < rc], the slab test of the first
 *    pulse of d; px = floor(fl(rc * fl32(1/c))) is the x index of the cell
 *    holding the cut; class = 7 - m (atoms that pass first) when cx - px is
 *    even in an even row or odd in an odd row, else class = m (atoms that
 *    pass last). So a cell that a slab cuts keeps the atoms that pulse sends
 *    together, and along a row such runs meet across neighbouring cells, and
 *    the cut cell's run meets the wholly selected cells below the cut;
 *  - force add order: pulses in reverse global order, plain fp32 adds in place.
 *
 * Layout: domain D = ix + nx * (iy + ny * iz) owns the slots
 * [base_D, base_D + ntotal_D) of one flat array of float3 records: first its
 * home atoms in sort order, then one contiguous region per pulse, in global
 * pulse order.
 *
 * All floating-point work is single IEEE binary32 operations, compiled with
 * -ffp-contract=off.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define DDHO_OK 0
#define DDHO_EINVAL (-1)
#define DDHO_ERANGE (-2)
#define DDHO_ENOMEM (-3)

#define DDHO_MAXP 64

typedef struct {
    int n[3];            /* domains per dimension; 0 = X, 1 = Y, 2 = Z */
    float L[3];          /* box edges (fp32) */
    float rc;            /* cutoff */
    float cell;          /* sort-cell edge; <= 0: one cell per domain */
    float *b[3];         /* boundaries, n[d] + 1 values per dimension */
    int ndom;
    int P;               /* total number of pulses */
    int pdim[DDHO_MAXP]; /* dimension of global pulse p */
    int pk[DDHO_MAXP];   /* index of pulse p inside its dimension */
    /* per domain */
    int *nhome;
    int *ntotal;
    int64_t *base;
    int **gid;           /* global atom id of every local slot */
    float **x;           /* local coordinates, 3 floats per slot */
    /* per (sender S, pulse p), index S * P + p */
    int *send;           /* number of map entries */
    int *split;          /* entries below the sender's home count */
    int *recv;           /* receiving domain R */
    int *roff;           /* first slot of the region at R */
    int *shift;          /* 1 when component pdim[p] gets + L */
    int **map;           /* sender-local slot indices, increasing */
} oplan;

/* ---------------------------------------------------------------- helpers */

static void dom_coords(const oplan *o, int D, int c[3])
{
    c[0] = D % o->n[0];
    c[1] = (D / o->n[0]) % o->n[1];
    c[2] = D / (o->n[0] * o->n[1]);
}

static int dom_index(const oplan *o, const int c[3])
{
    return c[0] + o->n[0] * (c[1] + o->n[1] * c[2]);
}

/* Receiver of S in a pulse along dimension d: the neighbour at index - 1. */
static int receiver_of(const oplan *o, int S, int d)
{
    int c[3];
    dom_coords(o, S, c);
    c[d] = (c[d] - 1 + o->n[d]) % o->n[d];
    return dom_index(o, c);
}

/* The unique i with b[i] <= v < b[i+1], found by a plain scan. */
static int interval_of(const float *b, int n, float v)
{
    for (int i = 0; i < n; i++)
        if (b[i] <= v && v < b[i + 1])
            return i;
    return -1;
}

static int grow(void **p, size_t nbytes)
{
    void *q = realloc(*p, nbytes ? nbytes : 1);
    if (!q)
        return DDHO_ENOMEM;
    *p = q;
    return DDHO_OK;
}

/* ------------------------------------------------------------ cell sort */

typedef struct {
    int64_t key;
    int cls;
    int gid;
} keyed;

static int cmp_keyed(const void *a, const void *b)
{
    const keyed *p = (const keyed *)a, *q = (const keyed *)b;
    if (p->key != q->key)
        return p->key < q->key ? -1 : 1;
    if (p->cls != q->cls)
        return p->cls < q->cls ? -1 : 1;
    return p->gid < q->gid ? -1 : (p->gid > q->gid ? 1 : 0);
}

/* Number of sort cells across [lo, hi) for edge c (at least one). */
static int cells_across(float lo, float hi, float c)
{
    if (!(c > 0.0f))
        return 1;
    int nc = (int)ceil(((double)hi - (double)lo) / (double)c);
    return nc < 1 ? 1 : nc;
}

static int cell_of(float v, float lo, float inv_c, int nc)
{
    if (nc == 1)
        return 0;
    float t = (v - lo) * inv_c;
    int ci = (int)floorf(t);
    if (ci < 0)
        ci = 0;
    if (ci > nc - 1)
        ci = nc - 1;
    return ci;
}

/* -------------------------------------------------------------- public API */

void ddho_free(void *h)
{
    oplan *o = (oplan *)h;
    if (!o)
        return;
    for (int d = 0; d < 3; d++)
        free(o->b[d]);
    if (o->gid)
        for (int D = 0; D < o->ndom; D++)
            free(o->gid[D]);
    if (o->x)
        for (int D = 0; D < o->ndom; D++)
            free(o->x[D]);
    if (o->map)
        for (int i = 0; i < o->ndom * o->P; i++)
            free(o->map[i]);
    free(o->gid);
    free(o->x);
    free(o->map);
    free(o->nhome);
    free(o->ntotal);
    free(o->base);
    free(o->send);
    free(o->split);
    free(o->recv);
    free(o->roff);
    free(o->shift);
    free(o);
}

/*
 * Pulse schedule only: fills pdim/pk and P, or returns DDHO_ERANGE.
 * Dimensions are visited Z, Y, X ("Accelerating GROMACS using
 * Device-initiated Remote Memory Access": phases Z -> Y -> X); a dimension
 * with one domain exchanges nothing.
 */
static int schedule(oplan *o)
{
    o->P = 0;
    for (int d = 2; d >= 0; d--) {
        if (o->n[d] == 1)
            continue;
        double wmin = 1e300, wmax = 0.0;
        for (int i = 0; i < o->n[d]; i++) {
            double w = (double)o->b[d][i + 1] - (double)o->b[d][i];
            if (w < wmin)
                wmin = w;
            if (w > wmax)
                wmax = w;
        }
        if ((double)o->rc > (double)o->L[d] - wmax)
            return DDHO_ERANGE;
        int np = 1;
        while ((double)np * wmin < (double)o->rc)
            np++;
        /* a relay chain longer than n_d - 1 would carry atoms back to their
           own domain (possible only within rounding of rc == L - w) */
        if (np > o->n[d] - 1)
            return DDHO_ERANGE;
        for (int k = 0; k < np; k++) {
            if (o->P >= DDHO_MAXP)
                return DDHO_ERANGE;
            o->pdim[o->P] = d;
            o->pk[o->P] = k;
            o->P++;
        }
    }
    return DDHO_OK;
}

static int setup_geometry(oplan *o, const int ndom[3], const float box[3], float rc, float cell)
{
    for (int d = 0; d < 3; d++) {
        if (ndom[d] < 1 || !(box[d] > 0.0f))
            return DDHO_EINVAL;
        o->n[d] = ndom[d];
        o->L[d] = box[d];
    }
    if (!(rc > 0.0f))
        return DDHO_EINVAL;
    o->rc = rc;
    o->cell = cell;
    for (int d = 0; d < 3; d++) {
        o->b[d] = (float *)malloc(sizeof(float) * (size_t)(o->n[d] + 1));
        if (!o->b[d])
            return DDHO_ENOMEM;
        for (int i = 0; i < o->n[d]; i++)
            o->b[d][i] = (float)((double)o->L[d] * (double)i / (double)o->n[d]);
        o->b[d][o->n[d]] = o->L[d];
    }
    o->ndom = o->n[0] * o->n[1] * o->n[2];
    return schedule(o);
}

/* Pulse schedule without atoms: number of pulses, or a negative error. */
int ddho_schedule(const int ndom[3], const float box[3], float rc, int *pdim, int *pk)
{
    oplan *o = (oplan *)calloc(1, sizeof(oplan));
    if (!o)
        return DDHO_ENOMEM;
    int rcode = setup_geometry(o, ndom, box, rc, 0.0f);
    int P = o->P;
    if (rcode == DDHO_OK)
        for (int p = 0; p < P; p++) {
            if (pdim)
                pdim[p] = o->pdim[p];
            if (pk)
                pk[p] = o->pk[p];
        }
    ddho_free(o);
    return rcode == DDHO_OK ? P : rcode;
}

/* Home assignment and cell sort of home atoms. */
static int assign_home(oplan *o, const float *xg, int n_atoms)
{
    int *dom_of = (int *)malloc(sizeof(int) * (size_t)(n_atoms > 0 ? n_atoms : 1));
    if (!dom_of)
        return DDHO_ENOMEM;
    for (int a = 0; a < n_atoms; a++) {
        int c[3];
        for (int d = 0; d < 3; d++) {
            float v = xg[3 * (size_t)a + d];
            if (!(v >= 0.0f && v < o->L[d])) {
                free(dom_of);
                return DDHO_EINVAL;
            }
            c[d] = interval_of(o->b[d], o->n[d], v);
            if (c[d] < 0) {
                free(dom_of);
                return DDHO_EINVAL;
            }
        }
        dom_of[a] = dom_index(o, c);
        o->nhome[dom_of[a]]++;
    }

    /* atoms of each domain, in increasing global id */
    int **members = (int **)calloc((size_t)o->ndom, sizeof(int *));
    int *fill = (int *)calloc((size_t)o->ndom, sizeof(int));
    if (!members || !fill) {
        free(members);
        free(fill);
        free(dom_of);
        return DDHO_ENOMEM;
    }
    for (int D = 0; D < o->ndom; D++) {
        members[D] = (int *)malloc(sizeof(int) * (size_t)(o->nhome[D] > 0 ? o->nhome[D] : 1));
        if (!members[D]) {
            for (int E = 0; E < D; E++)
                free(members[E]);
            free(members);
            free(fill);
            free(dom_of);
            return DDHO_ENOMEM;
        }
    }
    for (int a = 0; a < n_atoms; a++)
        members[dom_of[a]][fill[dom_of[a]]++] = a;

    float inv_c = o->cell > 0.0f ? (float)(1.0 / (double)o->cell) : 0.0f;
    const int px = (int)floorf(o->rc * inv_c);
    for (int D = 0; D < o->ndom; D++) {
        int c[3];
        dom_coords(o, D, c);
        float lo[3], hi[3];
        int nc[3];
        for (int d = 0; d < 3; d++) {
            lo[d] = o->b[d][c[d]];
            hi[d] = o->b[d][c[d] + 1];
            nc[d] = cells_across(lo[d], hi[d], o->cell);
        }
        const int m = o->nhome[D];
        keyed *list = (keyed *)malloc(sizeof(keyed) * (size_t)(m > 0 ? m : 1));
        o->ntotal[D] = m;
        o->gid[D] = (int *)malloc(sizeof(int) * (size_t)(m > 0 ? m : 1));
        o->x[D] = (float *)malloc(sizeof(float) * 3 * (size_t)(m > 0 ? m : 1));
        if (!list || !o->gid[D] || !o->x[D]) {
            free(list);
            for (int E = 0; E < o->ndom; E++)
                free(members[E]);
            free(members);
            free(fill);
            free(dom_of);
            return DDHO_ENOMEM;
        }
        for (int j = 0; j < m; j++) {
            const int a = members[D][j];
            int ci[3];
            for (int d = 0; d < 3; d++)
                ci[d] = cell_of(xg[3 * (size_t)a + d], lo[d], inv_c, nc[d]);
            const int64_t row = (int64_t)ci[1] + (int64_t)nc[1] * ci[2];
            const int odd = (int)(row % 2);
            list[j].key = (int64_t)(odd ? nc[0] - 1 - ci[0] : ci[0]) + (int64_t)nc[0] * row;
            int m = 0;
            for (int d = 0; d < 3; d++)
                if (xg[3 * (size_t)a + d] - lo[d] < o->rc)
                    m |= 1 << d;
            const int even_from_cut = (ci[0] - px) % 2 == 0;
            list[j].cls = even_from_cut != odd ? 7 - m : m;
            list[j].gid = a;
        }
        qsort(list, (size_t)m, sizeof(keyed), cmp_keyed);
        for (int j = 0; j < m; j++) {
            o->gid[D][j] = list[j].gid;
            for (int d = 0; d < 3; d++)
                o->x[D][3 * (size_t)j + d] = xg[3 * (size_t)list[j].gid + d];
        }
        free(list);
    }
    for (int D = 0; D < o->ndom; D++)
        free(members[D]);
    free(members);
    free(fill);
    free(dom_of);
    return DDHO_OK;
}

/*
 * One pulse of the first coordinate pass: choose every sender's map from its
 * current slots, then deliver the selected records to the receivers. All maps
 * of the pulse are chosen before any delivery, so a sender never forwards a
 * record in the same pulse in which it received it.
 */
static int run_pulse(oplan *o, int p)
{
    const int d = o->pdim[p];
    const int k = o->pk[p];
    const int P = o->P;

    /* 1. selection, per sender */
    for (int S = 0; S < o->ndom; S++) {
        int c[3];
        dom_coords(o, S, c);
        const float lo = o->b[d][c[d]];
        int first, last;
        if (k == 0) {
            first = 0;
            last = o->ntotal[S];
        } else {
            /* slots S received in the previous pulse of this dimension */
            int Q = -1;
            for (int T = 0; T < o->ndom; T++)
                if (o->recv[T * P + (p - 1)] == S)
                    Q = T;
            first = o->roff[Q * P + (p - 1)];
            last = first + o->send[Q * P + (p - 1)];
        }
        int *m = (int *)malloc(sizeof(int) * (size_t)(last - first > 0 ? last - first : 1));
        if (!m)
            return DDHO_ENOMEM;
        int cnt = 0, below = 0;
        for (int j = first; j < last; j++) {
            float dist = o->x[S][3 * (size_t)j + d] - lo;
            if (dist < o->rc) {
                m[cnt++] = j;
                if (j < o->nhome[S])
                    below++;
            }
        }
        o->map[S * P + p] = m;
        o->send[S * P + p] = cnt;
        o->split[S * P + p] = below;
        o->recv[S * P + p] = receiver_of(o, S, d);
        o->shift[S * P + p] = (c[d] == 0);
    }

    /* 2. delivery: the region lands right after the receiver's current slots */
    for (int S = 0; S < o->ndom; S++) {
        const int R = o->recv[S * P + p];
        const int cnt = o->send[S * P + p];
        const int off = o->ntotal[R];
        o->roff[S * P + p] = off;
        int need = off + cnt;
        if (grow((void **)&o->gid[R], sizeof(int) * (size_t)(need > 0 ? need : 1)) ||
            grow((void **)&o->x[R], sizeof(float) * 3 * (size_t)(need > 0 ? need : 1)))
            return DDHO_ENOMEM;
        const int *m = o->map[S * P + p];
        for (int i = 0; i < cnt; i++) {
            int j = m[i];
            o->gid[R][off + i] = o->gid[S][j];
            for (int e = 0; e < 3; e++) {
                float v = o->x[S][3 * (size_t)j + e];
                if (e == d && o->shift[S * P + p])
                    v = v + o->L[d];
                o->x[R][3 * (size_t)(off + i) + e] = v;
            }
        }
        o->ntotal[R] = need;
    }
    return DDHO_OK;
}

/*
 * Build the exchange plan from global positions xg[n_atoms][3] (all inside
 * [0, L)). On success *out holds the plan and 0 is returned; otherwise a
 * negative code (DDHO_EINVAL, DDHO_ERANGE, DDHO_ENOMEM).
 */
int ddho_build(const float *xg, int n_atoms, const int ndom[3], const float box[3],
               float rc, float cell, void **out)
{
    *out = NULL;
    if (n_atoms < 0 || (n_atoms > 0 && !xg))
        return DDHO_EINVAL;
    oplan *o = (oplan *)calloc(1, sizeof(oplan));
    if (!o)
        return DDHO_ENOMEM;
    int rcode = setup_geometry(o, ndom, box, rc, cell);
    if (rcode) {
        ddho_free(o);
        return rcode;
    }
    const int N = o->ndom, P = o->P;
    const int NP = N * P > 0 ? N * P : 1;
    o->nhome = (int *)calloc((size_t)N, sizeof(int));
    o->ntotal = (int *)calloc((size_t)N, sizeof(int));
    o->base = (int64_t *)calloc((size_t)N, sizeof(int64_t));
    o->gid = (int **)calloc((size_t)N, sizeof(int *));
    o->x = (float **)calloc((size_t)N, sizeof(float *));
    o->send = (int *)calloc((size_t)NP, sizeof(int));
    o->split = (int *)calloc((size_t)NP, sizeof(int));
    o->recv = (int *)calloc((size_t)NP, sizeof(int));
    o->roff = (int *)calloc((size_t)NP, sizeof(int));
    o->shift = (int *)calloc((size_t)NP, sizeof(int));
    o->map = (int **)calloc((size_t)NP, sizeof(int *));
    if (!o->nhome || !o->ntotal || !o->base || !o->gid || !o->x || !o->send || !o->split ||
        !o->recv || !o->roff || !o->shift || !o->map) {
        ddho_free(o);
        return DDHO_ENOMEM;
    }
    rcode = assign_home(o, xg, n_atoms);
    for (int p = 0; rcode == DDHO_OK && p < P; p++)
        rcode = run_pulse(o, p);
    if (rcode) {
        ddho_free(o);
        return rcode;
    }
    int64_t acc = 0;
    for (int D = 0; D < N; D++) {
        o->base[D] = acc;
        acc += o->ntotal[D];
    }
    *out = o;
    return DDHO_OK;
}

int ddho_ndomains(const void *h) { return ((const oplan *)h)->ndom; }
int ddho_npulses(const void *h) { return ((const oplan *)h)->P; }

int64_t ddho_nslots(const void *h)
{
    const oplan *o = (const oplan *)h;
    return o->ndom ? o->base[o->ndom - 1] + o->ntotal[o->ndom - 1] : 0;
}

void ddho_pulse_table(const void *h, int *pdim, int *pk)
{
    const oplan *o = (const oplan *)h;
    for (int p = 0; p < o->P; p++) {
        pdim[p] = o->pdim[p];
        pk[p] = o->pk[p];
    }
}

void ddho_bounds(const void *h, int d, float *out)
{
    const oplan *o = (const oplan *)h;
    for (int i = 0; i <= o->n[d]; i++)
        out[i] = o->b[d][i];
}

void ddho_domain_table(const void *h, int64_t *base, int *nhome, int *ntotal)
{
    const oplan *o = (const oplan *)h;
    for (int D = 0; D < o->ndom; D++) {
        base[D] = o->base[D];
        nhome[D] = o->nhome[D];
        ntotal[D] = o->ntotal[D];
    }
}

/* Per (S, p) tables, index S * P + p. */
void ddho_item_table(const void *h, int *send, int *split, int *recv, int *roff, int *shift)
{
    const oplan *o = (const oplan *)h;
    for (int i = 0; i < o->ndom * o->P; i++) {
        send[i] = o->send[i];
        split[i] = o->split[i];
        recv[i] = o->recv[i];
        roff[i] = o->roff[i];
        shift[i] = o->shift[i];
    }
}

/* All maps, concatenated in (S, p) order (S outer). */
void ddho_maps(const void *h, int *out)
{
    const oplan *o = (const oplan *)h;
    int64_t pos = 0;
    for (int i = 0; i < o->ndom * o->P; i++) {
        memcpy(out + pos, o->map[i], sizeof(int) * (size_t)o->send[i]);
        pos += o->send[i];
    }
}

/* Global atom id of every slot of the flat layout. */
void ddho_slot_ids(const void *h, int *out)
{
    const oplan *o = (const oplan *)h;
    for (int D = 0; D < o->ndom; D++)
        memcpy(out + o->base[D], o->gid[D], sizeof(int) * (size_t)o->ntotal[D]);
}

/* Flat coordinates after the first (map-building) pass. */
void ddho_coords(const void *h, float *out)
{
    const oplan *o = (const oplan *)h;
    for (int D = 0; D < o->ndom; D++)
        memcpy(out + 3 * o->base[D], o->x[D], sizeof(float) * 3 * (size_t)o->ntotal[D]);
}

/*
 * Coordinate pass with the maps fixed: pulses in increasing global order
 * (Z, then Y, then X); for every sender S and entry i the record
 * x[base_S + map[i]] is copied to x[base_R + roff + i], with + L_d on the
 * pulse's component when the sender sits at index 0. Reads home slots and
 * earlier regions only, writes every halo slot.
 */
void ddho_exchange_coords(const void *h, float *xf, int nthreads)
{
    const oplan *o = (const oplan *)h;
    const int P = o->P;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (int p = 0; p < P; p++) {
        const int d = o->pdim[p];
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (nthreads > 1)
#endif
        for (int S = 0; S < o->ndom; S++) {
            const int it = S * P + p;
            const int R = o->recv[it];
            const int64_t src = o->base[S];
            const int64_t dst = o->base[R] + o->roff[it];
            const int *m = o->map[it];
            for (int i = 0; i < o->send[it]; i++) {
                for (int e = 0; e < 3; e++) {
                    float v = xf[3 * (src + m[i]) + e];
                    if (e == d && o->shift[it])
                        v = v + o->L[d];
                    xf[3 * (dst + i) + e] = v;
                }
            }
        }
    }
}

/*
 * Force pass: pulses in decreasing global order (X, then Y, then Z); for every
 * sender S and entry i, f[base_S + map[i]] += f[base_R + roff + i] (fp32 add,
 * in place). Within one pulse the writes (the sender's home slots and earlier
 * regions) never overlap the reads (the receivers' region of this pulse), and
 * map entries are unique, so the order inside a pulse does not matter.
 */
void ddho_exchange_forces(const void *h, float *ff, int nthreads)
{
    const oplan *o = (const oplan *)h;
    const int P = o->P;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (int p = P - 1; p >= 0; p--) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (nthreads > 1)
#endif
        for (int S = 0; S < o->ndom; S++) {
            const int it = S * P + p;
            const int R = o->recv[it];
            const int64_t dst = o->base[S];
            const int64_t src = o->base[R] + o->roff[it];
            const int *m = o->map[it];
            for (int i = 0; i < o->send[it]; i++)
                for (int e = 0; e < 3; e++)
                    ff[3 * (dst + m[i]) + e] = ff[3 * (dst + m[i]) + e] + ff[3 * (src + i) + e];
        }
    }
}
